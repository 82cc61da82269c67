// Part 3 of the whole-plane variant table.
#include "wtconv_plane_variant.h"

namespace wtc {

// Six levels on 64 x 64, and L = 0: the plain 7 x 7 depthwise conv
// baseline on the stage shapes (and a small edge case).
const PlaneVariant* plane_table_3(int* n) {
    static const PlaneVariant table[] = {
        WTC_PLANE_ROW(5, 6, 64, 64, 1, 512)
        WTC_PLANE_ROW(7, 0, 56, 56, 1, 256)
        WTC_PLANE_ROW(7, 0, 28, 28, 4, 256)
        WTC_PLANE_ROW(7, 0, 14, 14, 8, 256)
        WTC_PLANE_ROW(7, 0, 12, 20, 2, 256)
    };
    *n = int(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace wtc
