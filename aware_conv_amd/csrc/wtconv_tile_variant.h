// Host-side description of one instantiated tile-kernel family (large planes:
// TH x TW output tiles, the base conv and LT levels per tile).
#pragma once

#include "wtconv_kernels.h"

namespace wtc {

struct TileVariant {
    int K, LT, dtype, TH, TW, NT;
    const void* fwd;
    const void* bwi;
    const void* bww;
    const void* bwd;  // fused backward: input gradient and weight partials
    size_t lds_apply, lds_bww, lds_bwd;
};

constexpr int kTileH = 32, kTileW = 32, kTileNT = 256;

template <int K, int LT, typename T>
TileVariant make_tile_variant(int dtype) {
    using G = dev::Geo<K, LT, kTileH, kTileW, 1, kTileNT, LT>;
    return TileVariant{
        K, LT, dtype, kTileH, kTileW, kTileNT,
        reinterpret_cast<const void*>(&dev::k_tile_apply<K, LT, kTileH, kTileW, kTileNT, T, false>),
        reinterpret_cast<const void*>(&dev::k_tile_apply<K, LT, kTileH, kTileW, kTileNT, T, true>),
        reinterpret_cast<const void*>(&dev::k_tile_bww<K, LT, kTileH, kTileW, kTileNT, T>),
        reinterpret_cast<const void*>(&dev::k_tile_bwd<K, LT, kTileH, kTileW, kTileNT, T>),
        dev::apply_lds_bytes<G>(), dev::bww_lds_bytes<G>(), dev::tile_bwd_lds_bytes<G>()};
}

// Tables of the per-k translation units (LT = 1, 2, 3; fp32 and fp16).
const TileVariant* tile_table_k1(int* n);
const TileVariant* tile_table_k3(int* n);
const TileVariant* tile_table_k5(int* n);
const TileVariant* tile_table_k7(int* n);

}  // namespace wtc
