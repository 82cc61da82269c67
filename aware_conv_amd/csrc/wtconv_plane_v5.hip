// Part 5 of the whole-plane variant table.
#include "wtconv_plane_variant.h"

namespace wtc {

// The sides that stage shapes with more levels are zero-extended to: 28 at
// three levels -> 32, 14 at two -> 16, 7 at two or three -> 8.
const PlaneVariant* plane_table_5(int* n) {
    static const PlaneVariant table[] = {
        WTC_PLANE_ROW(5, 3, 32, 32, 1, 256)
        WTC_PLANE_ROW(5, 2, 16, 16, 4, 256)
        WTC_PLANE_ROW(5, 2, 8, 8, 8, 256)
        WTC_PLANE_ROW(5, 3, 8, 8, 8, 256)
    };
    *n = int(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace wtc
