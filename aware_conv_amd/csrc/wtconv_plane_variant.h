// Variant table of the whole-plane kernels: one row per (K, L, H, W, dtype)
// this build instantiates, split over several translation units so that
// they compile in parallel.
#pragma once

#include "wtconv_kernels.h"

namespace wtc {

struct PlaneVariant {
    int K, L, H, W, dtype, P, NT;
    const void* fwd;
    const void* bwi;
    const void* bww;
    const void* bwd;        // fused backward, NULL where its LDS does not fit
    const void* bwd_cross;  // the same, for ranges that span channels
    size_t lds_apply, lds_bww, lds_bwd;
};

constexpr size_t kPlaneMaxLds = 163840;  // LDS of one gfx950 compute unit

template <int K, int L, int H, int W, int P, int NT, typename T>
PlaneVariant make_plane_variant(int dtype) {
    using namespace dev;
    using G = Geo<K, L, H, W, P, NT>;
    using GG = GeoGrad<K, L, H, W, P, NT>;
    const size_t la = apply_lds_bytes<G>();
    const size_t lb = bww_lds_bytes<GG>();
    constexpr size_t ld = bwd_lds_bytes<GG>();
    const void* fused = nullptr;
    const void* fused_cross = nullptr;
    if constexpr (ld <= kPlaneMaxLds) {
        fused = reinterpret_cast<const void*>(&k_plane_bwd<K, L, H, W, P, NT, T, false>);
        fused_cross = reinterpret_cast<const void*>(&k_plane_bwd<K, L, H, W, P, NT, T, true>);
    }
    return PlaneVariant{K, L, H, W, dtype, P, NT,
                        reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, false>),
                        reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, true>),
                        reinterpret_cast<const void*>(&k_plane_bww<K, L, H, W, P, NT, T>),
                        fused, fused_cross, la, lb, ld};
}

// Rows (K, L, H, W, planes per group, threads), both dtypes each.
#define WTC_PLANE_ROW(K, L, H, W, P, NT) make_plane_variant<K, L, H, W, P, NT, float>(WTCONV_F32), \
                                         make_plane_variant<K, L, H, W, P, NT, __half>(WTCONV_F16),

// The parts of the table, one per translation unit.
const PlaneVariant* plane_table_0(int* n);
const PlaneVariant* plane_table_1(int* n);
const PlaneVariant* plane_table_2(int* n);
const PlaneVariant* plane_table_3(int* n);

}  // namespace wtc
