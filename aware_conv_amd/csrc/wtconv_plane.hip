// Whole-plane kernels of the fused WTConv layer: variant lookup, launch
// sizing and the host entry points for shapes whose planes fit LDS.
#include "wtconv_plane_variant.h"

namespace wtc {
namespace {
using namespace dev;

using Variant = PlaneVariant;

const Variant* find_variant(const wtconv_shape& s) {
    const PlaneVariant* (*parts[])(int*) = {plane_table_0, plane_table_1, plane_table_2,
                                            plane_table_3, plane_table_4, plane_table_5};
    for (auto part : parts) {
        int n = 0;
        const Variant* t = part(&n);
        for (int i = 0; i < n; ++i)
            if (t[i].K == s.k && t[i].L == s.L && t[i].H == s.H && t[i].W == s.W &&
                t[i].dtype == s.dtype)
                return &t[i];
    }
    return nullptr;
}

hipError_t prepare(const void* fn, size_t lds) { return prepare_lds(fn, lds); }

// Weight gradient: chunks of the batch per channel.  At most this many, so
// that the workspace size is a function of the shape alone.
constexpr int kMaxChunks = 64;

int bww_chunks(const wtconv_shape& s, int P, int slots) {
    const int ngroups = cdiv(s.B, P);
    int want = slots / (s.C > 0 ? s.C : 1);
    if (want < 1) want = 1;
    if (want > kMaxChunks) want = kMaxChunks;
    if (want > ngroups) want = ngroups;
    const int gpw = cdiv(ngroups, want);
    return cdiv(ngroups, gpw);
}

// The kernel set for planes stored as `rg`.
const PlaneKernels& kernels_for(const Variant* v, Rag rg) {
    return (rg.Hs == v->H && rg.Ws == v->W) ? v->full : v->rag;
}

}  // namespace

bool plane_supported(const wtconv_shape& s) {
    const Variant* v = find_variant(s);
    if (!v) return false;
    // buffer offsets within a group (P planes of one channel, C planes
    // apart) are 32-bit: larger shapes take the tile path
    const size_t esz = s.dtype == WTCONV_F32 ? 4 : 2;
    return size_t(v->P) * size_t(s.C) * size_t(s.H) * size_t(s.W) * esz < (size_t(1) << 31);
}

// Fused backward: workgroups over balanced ranges of (channel, group)
// items, at most this many (a compute unit holds at most 8 of them).
constexpr int kMaxBwdWGs = 2048;

// Upper bound of the partial rows per channel of the fused backward for any
// workgroup count up to kMaxBwdWGs (ranges of at least floor(T / nwg) items).
int bwd_rows_bound(const wtconv_shape& s, int P) {
    const long ng = cdiv(s.B, P), total = ng * s.C;
    const long nwg = total < kMaxBwdWGs ? total : kMaxBwdWGs;
    const long per = total / (nwg > 0 ? nwg : 1);
    long r = (ng + per - 1) / (per > 0 ? per : 1) + 1;
    if (r > ng) r = ng;
    return int(r);
}

size_t plane_workspace_bytes(const wtconv_shape& s) {
    const Variant* v = find_variant(s);
    if (!v || s.B == 0 || s.C == 0) return 0;
    const int ngroups = cdiv(s.B, v->P);
    const int nchunk = ngroups < kMaxChunks ? ngroups : kMaxChunks;
    const int rows = nchunk > bwd_rows_bound(s, v->P) ? nchunk : bwd_rows_bound(s, v->P);
    const int KK = s.k * s.k;
    const size_t npart = size_t(KK) + 1 + size_t(4) * s.L * KK;
    return size_t(rows) * s.C * npart * sizeof(float);
}

hipError_t plane_apply(const wtconv_shape& s, const void* in, const Params& p, void* out,
                       bool flip, hipStream_t stream, Rag rg) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    const PlaneKernels& ks = kernels_for(v, rg);
    const void* fn = flip ? ks.bwi : ks.fwd;
    hipError_t e = prepare(fn, v->lds_apply);
    if (e != hipSuccess) return e;
    int B = s.B, C = s.C;
    const long total = long(cdiv(s.B, v->P)) * s.C;
    long nwg = resident_wgs(fn, v->NT, v->lds_apply);
    if (nwg > total) nwg = total;
    // as few workgroups as take the same most groups each: with 3072 groups
    // on 1280 slots, 1024 workgroups of three instead of 512 of three and
    // 768 of two (the last round then runs on every workgroup, not 40%)
    if (nwg > 0) {
        const long per = (total + nwg - 1) / nwg;
        nwg = (total + per - 1) / per;
    }
    const void* bb = flip ? p.w_base : p.b_base;  // read but unused when flipped
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    void* args[] = {&in, &wb, &bb, &sb, &ww, &sw, &out, &B, &C, &rg};
    e = hipLaunchKernel(fn, dim3(unsigned(nwg)), dim3(v->NT), args, v->lds_apply, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

namespace {
template <typename T, int K>
hipError_t launch_final_k(const wtconv_shape& s, const float* part, int nchunk,
                          const LinearRows& rows, const Params& p, const Grads& g,
                          hipStream_t stream) {
    // fp64 row sums [NPART], fp32 filters [KK + 4 L KK], scales [4 L],
    // beta and the bias
    const size_t KK = size_t(K) * K, L = size_t(s.L);
    const size_t lds = sizeof(double) * (KK + 1 + 4 * L * KK) +
                       sizeof(float) * (KK + 4 * L * KK + 4 * L + 2);
    // idle waves would still cost their launch and the barrier
    const unsigned nt = unsigned(bww_final_threads(K, s.L));
    hipLaunchKernelGGL((k_bww_final<T, K>), dim3(s.C), dim3(nt), lds, stream, part, nchunk,
                       rows, s.C, s.L, (const T*)p.w_base, (const T*)p.b_base,
                       (const T*)p.s_base, (const T*)p.w_wav, (const T*)p.s_wav,
                       (T*)g.dw_base, (T*)g.db_base, (T*)g.ds_base, (T*)g.dw_wav, (T*)g.ds_wav);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_final(const wtconv_shape& s, const float* part, int nchunk,
                        const LinearRows& rows, const Params& p, const Grads& g,
                        hipStream_t stream) {
    switch (s.k) {
        case 1: return launch_final_k<T, 1>(s, part, nchunk, rows, p, g, stream);
        case 3: return launch_final_k<T, 3>(s, part, nchunk, rows, p, g, stream);
        case 5: return launch_final_k<T, 5>(s, part, nchunk, rows, p, g, stream);
        case 7: return launch_final_k<T, 7>(s, part, nchunk, rows, p, g, stream);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t finalize_grads(const wtconv_shape& s, const float* part, int rows, const Params& p,
                          const Grads& g, hipStream_t stream) {
    const LinearRows none{1, 0, 0, 0};
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, part, rows, none, p, g, stream)
                                 : launch_final<__half>(s, part, rows, none, p, g, stream);
}

namespace {
// The fused backward's launch (kernels of the LinearRows family: k_plane_bwd,
// k_plane_bwd1, with or without dx): workgroups over balanced ranges of
// (channel, group) items, then the finalize over each channel's rows.
hipError_t launch_linear(const wtconv_shape& s, const Variant* v, const void* fn_one,
                         const void* fn_cross, const void* x, const void* dy, const Params& p,
                         void* dx, const Grads& g, void* workspace, hipStream_t stream,
                         Rag rg) {
    hipError_t e = prepare(fn_one, v->lds_bwd);
    if (e != hipSuccess) return e;
    const int ngroups = cdiv(s.B, v->P);
    const long total = long(ngroups) * s.C;
    long nwg = resident_wgs(fn_one, v->NT, v->lds_bwd);
    if (nwg > kMaxBwdWGs) nwg = kMaxBwdWGs;
    // a multiple of C puts every range inside one channel, which the kernel
    // without mid-range reductions runs faster: take it when it keeps at
    // least 7/8 of the resident slots (or covers every item)
    const long per_c = nwg / s.C;
    bool cross = true;
    if (per_c >= 1 && per_c * s.C * 8 >= nwg * 7) {
        nwg = per_c * s.C;
        cross = false;
    }
    if (nwg >= total) {
        nwg = total;  // one item per range: inside one channel
        cross = false;
    }
    LinearRows rows{total, int(nwg), ngroups, 0};
    for (int c = 0; c < s.C; ++c)
        if (rows.count(c) > rows.rmax) rows.rmax = rows.count(c);
    if (rows.rmax > bwd_rows_bound(s, v->P)) return hipErrorInvalidValue;  // workspace
    int B = s.B, C = s.C;
    float* part = static_cast<float*>(workspace);
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    void* args[] = {&x, &dy, &wb, &sb, &ww, &sw, &dx, &part, &B, &C, &rows, &rg};
    const void* fn = cross ? fn_cross : fn_one;
    if (cross && (e = prepare(fn, v->lds_bwd)) != hipSuccess) return e;
    e = hipLaunchKernel(fn, dim3(unsigned(nwg)), dim3(v->NT), args, v->lds_bwd, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, part, 0, rows, p, g, stream)
                                 : launch_final<__half>(s, part, 0, rows, p, g, stream);
}
}  // namespace

hipError_t plane_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                            const Params& p, const Grads& g, void* workspace,
                            hipStream_t stream, Rag rg) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    const PlaneKernels& ks = kernels_for(v, rg);
    // shapes with the one-side fused backward take its weight-only form
    if (ks.bww1)
        return launch_linear(s, v, ks.bww1, ks.bww1_cross, x, dy, p, nullptr, g, workspace,
                             stream, rg);
    hipError_t e = prepare(ks.bww, v->lds_bww);
    if (e != hipSuccess) return e;
    const int nchunk = bww_chunks(s, v->P, resident_wgs(ks.bww, v->NT, v->lds_bww));
    int gpw = cdiv(cdiv(s.B, v->P), nchunk), B = s.B, C = s.C;
    float* part = static_cast<float*>(workspace);
    void* args[] = {&x, &dy, &part, &B, &C, &gpw, &rg};
    e = hipLaunchKernel(ks.bww, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                        v->lds_bww, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    return finalize_grads(s, part, nchunk, p, g, stream);
}

hipError_t plane_bwd(const wtconv_shape& s, const void* x, const void* dy, const Params& p,
                     void* dx, const Grads& g, void* workspace, hipStream_t stream, Rag rg) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    const PlaneKernels& ks = kernels_for(v, rg);
    if (!ks.bwd) {
        hipError_t e = plane_apply(s, dy, p, dx, true, stream, rg);
        if (e != hipSuccess) return e;
        return plane_bwd_weight(s, x, dy, p, g, workspace, stream, rg);
    }
    return launch_linear(s, v, ks.bwd, ks.bwd_cross, x, dy, p, dx, g, workspace, stream, rg);
}

hipError_t zero_grads(const wtconv_shape& s, const Params& p, const Grads& g,
                      hipStream_t stream) {
    return finalize_grads(s, nullptr, 0, p, g, stream);
}

}  // namespace wtc
