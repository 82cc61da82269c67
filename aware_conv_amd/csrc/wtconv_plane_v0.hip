// Part 0 of the whole-plane variant table.
#include "wtconv_plane_variant.h"

namespace wtc {

// The ConvNeXt-T stage shapes (the 7 x 7 planes of stage 4 run zero-extended
// to 8 x 8).  14 x 14 takes four planes per group on two waves: its 120 tiles
// fit 128 lanes and the fused backward's LDS lets five workgroups share a
// compute unit (eight planes on four waves: 2.5 workgroups of work per slot,
// the two-side backward at two per unit; 3-4% slower both ways).
const PlaneVariant* plane_table_0(int* n) {
    static const PlaneVariant table[] = {
        WTC_PLANE_ROW(5, 2, 56, 56, 1, 256)
        WTC_PLANE_ROW(5, 2, 28, 28, 2, 256)
        WTC_PLANE_ROW(5, 1, 14, 14, 4, 128)
        WTC_PLANE_ROW(5, 1, 8, 8, 16, 256)
        WTC_PLANE_ROW(5, 2, 32, 32, 1, 256)
    };
    *n = int(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace wtc
