// Variant table of the whole-plane kernels: one row per (K, L, H, W, dtype)
// this build instantiates, split over several translation units so that
// they compile in parallel.
#pragma once

#include "wtconv_kernels.h"

namespace wtc {

// The kernels of one shape, for planes stored at that shape or (`rag`) as
// smaller corners of it (Rag).
struct PlaneKernels {
    const void* fwd;
    const void* bwi;
    const void* bww;
    const void* bwd;        // fused backward, NULL where its LDS does not fit
    const void* bwd_cross;  // the same, for ranges that span channels
    const void* bww1;       // weight gradient alone on the one-side kernel, or NULL
    const void* bww1_cross;
};

struct PlaneVariant {
    int K, L, H, W, dtype, P, NT;
    PlaneKernels full, rag;
    size_t lds_apply, lds_bww, lds_bwd;
};

constexpr size_t kPlaneMaxLds = 163840;  // LDS of one gfx950 compute unit

// Which fused backward a shape takes.  The one-side kernel (x, then dy,
// through one set of arrays; one window per tile for the conv and the taps)
// has half the LDS and half the window reads of the two-side kernel but one
// more commit phase and two more barriers per group.  Measured on the stage
// shapes, it wins where a lane's tile holds at least 20 outputs (56 x 56:
// 28 outputs, 97.6 -> 89.2 us per backward) or where there are no wavelet
// levels (the plain depthwise conv: x's pass is a copy), and loses on the
// 14-output tiles of the 28 x 28 shape (56.0 -> 58.5 us; fp16 55.5 -> 56.9
// us with the wave priorities of both kernels), whose two-side LDS already
// lets three workgroups share a compute unit.
// Two small shapes are measured exceptions (B = 64, per fused backward):
// 14 x 14 at k = 5, L = 1 (four planes per group on 128 threads: 40.1 ->
// 36.7 us, fp16 41.0 -> 37.9 us; its 14-output tiles notwithstanding) and
// 8 x 8 at L = 3 (57.6 -> 47.0 us) take the one-side kernel; 8 x 8 at L = 1
// and 2 keep the two-side one (the one-side took 53.6 and 92.5 us against
// 39.7 and 46.3).
template <int K, int L, int H, int W, int P, int NT>
constexpr bool bwd_one_side() {
    using G = dev::Geo<K, L, H, W, P, NT>;
    constexpr bool measured = (K == 5 && L == 1 && H == 14 && W == 14) ||
                              (K == 5 && L == 3 && H == 8 && W == 8);
    return (L == 0 || G::Q * G::R >= 20 || measured) && dev::bwd1_lds_bytes<G>() <= kPlaneMaxLds;
}

template <int K, int L, int H, int W, int P, int NT, typename T, bool RAG>
PlaneKernels make_plane_kernels() {
    using namespace dev;
    using G = Geo<K, L, H, W, P, NT>;
    using GG = GeoGrad<K, L, H, W, P, NT>;
    constexpr bool one_side = bwd_one_side<K, L, H, W, P, NT>();
    constexpr size_t ld = one_side ? bwd1_lds_bytes<G>() : bwd_lds_bytes<GG>();
    auto fn = [](auto f) { return reinterpret_cast<const void*>(f); };
    PlaneKernels k{fn(&k_plane_apply<K, L, H, W, P, NT, T, false, RAG>),
                   fn(&k_plane_apply<K, L, H, W, P, NT, T, true, RAG>),
                   fn(&k_plane_bww<K, L, H, W, P, NT, T, RAG>),
                   nullptr, nullptr, nullptr, nullptr};
    if constexpr (one_side) {
        k.bwd = fn(&k_plane_bwd1<K, L, H, W, P, NT, T, false, true, RAG>);
        k.bwd_cross = fn(&k_plane_bwd1<K, L, H, W, P, NT, T, true, true, RAG>);
        k.bww1 = fn(&k_plane_bwd1<K, L, H, W, P, NT, T, false, false, RAG>);
        k.bww1_cross = fn(&k_plane_bwd1<K, L, H, W, P, NT, T, true, false, RAG>);
    } else if constexpr (ld <= kPlaneMaxLds) {
        k.bwd = fn(&k_plane_bwd<K, L, H, W, P, NT, T, false, RAG>);
        k.bwd_cross = fn(&k_plane_bwd<K, L, H, W, P, NT, T, true, RAG>);
    }
    return k;
}

template <int K, int L, int H, int W, int P, int NT, typename T>
PlaneVariant make_plane_variant(int dtype) {
    using namespace dev;
    using G = Geo<K, L, H, W, P, NT>;
    using GG = GeoGrad<K, L, H, W, P, NT>;
    constexpr bool one_side = bwd_one_side<K, L, H, W, P, NT>();
    constexpr size_t ld = one_side ? bwd1_lds_bytes<G>() : bwd_lds_bytes<GG>();
    return PlaneVariant{K, L, H, W, dtype, P, NT,
                        make_plane_kernels<K, L, H, W, P, NT, T, false>(),
                        make_plane_kernels<K, L, H, W, P, NT, T, true>(),
                        apply_lds_bytes<G>(), bww_lds_bytes<GG>(), ld};
}

// Rows (K, L, H, W, planes per group, threads), both dtypes each.
#define WTC_PLANE_ROW(K, L, H, W, P, NT) make_plane_variant<K, L, H, W, P, NT, float>(WTCONV_F32), \
                                         make_plane_variant<K, L, H, W, P, NT, __half>(WTCONV_F16),

// The parts of the table, one per translation unit.
const PlaneVariant* plane_table_0(int* n);
const PlaneVariant* plane_table_1(int* n);
const PlaneVariant* plane_table_2(int* n);
const PlaneVariant* plane_table_3(int* n);
const PlaneVariant* plane_table_4(int* n);
const PlaneVariant* plane_table_5(int* n);

}  // namespace wtc
