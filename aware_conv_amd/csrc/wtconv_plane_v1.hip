// Part 1 of the whole-plane variant table.
#include "wtconv_plane_variant.h"

namespace wtc {

// Small shapes for edge cases.
const PlaneVariant* plane_table_1(int* n) {
    static const PlaneVariant table[] = {
        WTC_PLANE_ROW(1, 1, 8, 8, 8, 256)
        WTC_PLANE_ROW(3, 1, 8, 8, 8, 256)
        WTC_PLANE_ROW(3, 2, 16, 16, 4, 256)
        WTC_PLANE_ROW(3, 3, 16, 16, 4, 256)
        WTC_PLANE_ROW(5, 3, 16, 16, 4, 256)
    };
    *n = int(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace wtc
