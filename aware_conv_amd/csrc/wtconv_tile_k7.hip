// Tile kernels for k = 7 (instantiated in a unit of their own so the kernel
// sizes compile in parallel).
#include <hip/hip_fp16.h>

#include "wtconv_tile_variant.h"

namespace wtc {

const TileVariant* tile_table_k7(int* n) {
    static const TileVariant t[] = {
        make_tile_variant<7, 1, float>(WTCONV_F32), make_tile_variant<7, 1, __half>(WTCONV_F16),
        make_tile_variant<7, 2, float>(WTCONV_F32), make_tile_variant<7, 2, __half>(WTCONV_F16),
        make_tile_variant<7, 3, float>(WTCONV_F32), make_tile_variant<7, 3, __half>(WTCONV_F16),
    };
    *n = int(sizeof(t) / sizeof(t[0]));
    return t;
}

}  // namespace wtc
