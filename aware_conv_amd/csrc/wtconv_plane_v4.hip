// Part 4 of the whole-plane variant table.
#include "wtconv_plane_variant.h"

namespace wtc {

// Other level counts at the ConvNeXt-T stage-1 and stage-2 sides.
const PlaneVariant* plane_table_4(int* n) {
    static const PlaneVariant table[] = {
        WTC_PLANE_ROW(5, 1, 56, 56, 1, 256)
        WTC_PLANE_ROW(5, 3, 56, 56, 1, 256)
        WTC_PLANE_ROW(5, 1, 28, 28, 2, 256)
    };
    *n = int(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace wtc
