// Part 2 of the whole-plane variant table.
#include "wtconv_plane_variant.h"

namespace wtc {

// Small shapes for edge cases: k = 7, H != W, deeper cascades.
const PlaneVariant* plane_table_2(int* n) {
    static const PlaneVariant table[] = {
        WTC_PLANE_ROW(7, 2, 16, 16, 4, 256)
        WTC_PLANE_ROW(7, 1, 14, 14, 8, 256)
        WTC_PLANE_ROW(3, 2, 16, 32, 2, 256)
        WTC_PLANE_ROW(5, 4, 32, 32, 1, 256)
        WTC_PLANE_ROW(3, 5, 32, 32, 1, 256)
    };
    *n = int(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace wtc
