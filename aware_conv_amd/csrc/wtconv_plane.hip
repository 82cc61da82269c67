// Whole-plane variants of the fused WTConv kernels: the variant table,
// launch sizing and the host entry points for shapes whose planes fit LDS.
#include "wtconv_kernels.h"

namespace wtc {
namespace {
using namespace dev;

struct Variant {
    int K, L, H, W, dtype, P, NT;
    const void* fwd;
    const void* bwi;
    const void* bww;
    const void* bwd;  // fused backward, NULL where its LDS does not fit
    size_t lds_apply, lds_bww, lds_bwd;
};

constexpr size_t kMaxLds = 163840;  // LDS of one gfx950 compute unit

template <int K, int L, int H, int W, int P, int NT, typename T>
Variant make_variant(int dtype) {
    using G = Geo<K, L, H, W, P, NT>;
    using GG = GeoGrad<K, L, H, W, P, NT>;
    const size_t la = apply_lds_bytes<G>();
    const size_t lb = bww_lds_bytes<GG>();
    constexpr size_t ld = bwd_lds_bytes<GG>();
    const void* fused = nullptr;
    if constexpr (ld <= kMaxLds)
        fused = reinterpret_cast<const void*>(&k_plane_bwd<K, L, H, W, P, NT, T>);
    return Variant{K, L, H, W, dtype, P, NT,
                   reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, false>),
                   reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, true>),
                   reinterpret_cast<const void*>(&k_plane_bww<K, L, H, W, P, NT, T>),
                   fused, la, lb, ld};
}

// (K, L, H, W, planes per group, threads).  The ConvNeXt-T stage shapes
// first, then small shapes for edge cases; L = 0 rows are the plain 7 x 7
// depthwise conv baseline on the stage shapes (and a small edge case).
#define WTC_PLANE_VARIANTS(X) \
    X(5, 2, 56, 56, 1, 256)   \
    X(5, 2, 28, 28, 2, 256)   \
    X(5, 1, 14, 14, 8, 256)   \
    X(5, 2, 32, 32, 1, 256)   \
    X(1, 1, 8, 8, 8, 256)     \
    X(3, 1, 8, 8, 8, 256)     \
    X(3, 2, 16, 16, 4, 256)   \
    X(3, 3, 16, 16, 4, 256)   \
    X(5, 3, 16, 16, 4, 256)   \
    X(7, 2, 16, 16, 4, 256)   \
    X(7, 1, 14, 14, 8, 256)   \
    X(3, 2, 16, 32, 2, 256)   \
    X(5, 4, 32, 32, 1, 256)   \
    X(3, 5, 32, 32, 1, 256)   \
    X(5, 6, 64, 64, 1, 512)   \
    X(7, 0, 56, 56, 1, 256)   \
    X(7, 0, 28, 28, 4, 256)   \
    X(7, 0, 14, 14, 8, 256)   \
    X(7, 0, 12, 20, 2, 256)

const Variant* find_variant(const wtconv_shape& s) {
    static const Variant table[] = {
#define WTC_X(K, L, H, W, P, NT) make_variant<K, L, H, W, P, NT, float>(WTCONV_F32), \
                                 make_variant<K, L, H, W, P, NT, __half>(WTCONV_F16),
        WTC_PLANE_VARIANTS(WTC_X)
#undef WTC_X
    };
    for (const Variant& v : table)
        if (v.K == s.k && v.L == s.L && v.H == s.H && v.W == s.W && v.dtype == s.dtype) return &v;
    return nullptr;
}

hipError_t prepare(const void* fn, size_t lds) {
    if (lds > 65536)
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    return hipSuccess;
}

// Workgroups that fit on the whole device at once for this kernel (compute
// units times resident workgroups per unit), 1024 when it cannot be queried.
int resident_wgs(const void* fn, int nt, size_t lds) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, nt, lds) != hipSuccess ||
        cus <= 0 || per <= 0)
        return 1024;
    return cus * per;
}

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

}  // namespace

bool plane_supported(const wtconv_shape& s) { return find_variant(s) != nullptr; }

size_t plane_workspace_bytes(const wtconv_shape& s) {
    const Variant* v = find_variant(s);
    if (!v || s.B == 0 || s.C == 0) return 0;
    const int ngroups = cdiv(s.B, v->P);
    const int nchunk = ngroups < kMaxChunks ? ngroups : kMaxChunks;
    const int KK = s.k * s.k;
    const size_t npart = size_t(KK) + 1 + size_t(4) * s.L * KK;
    return size_t(nchunk) * s.C * npart * sizeof(float);
}

hipError_t plane_apply(const wtconv_shape& s, const void* in, const Params& p, void* out,
                       bool flip, hipStream_t stream) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    const void* fn = flip ? v->bwi : v->fwd;
    hipError_t e = prepare(fn, v->lds_apply);
    if (e != hipSuccess) return e;
    int B = s.B, C = s.C;
    const long total = long(cdiv(s.B, v->P)) * s.C;
    long nwg = resident_wgs(fn, v->NT, v->lds_apply);
    if (nwg > total) nwg = total;
    const void* bb = flip ? p.w_base : p.b_base;  // unread when flipped
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    void* args[] = {&in, &wb, &bb, &sb, &ww, &sw, &out, &B, &C};
    e = hipLaunchKernel(fn, dim3(unsigned(nwg)), dim3(v->NT), args, v->lds_apply, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

namespace {
template <typename T>
hipError_t launch_final(const wtconv_shape& s, const float* part, int nchunk, const Params& p,
                        const Grads& g, hipStream_t stream) {
    const int KK = s.k * s.k;
    const size_t lds = sizeof(float) * (size_t(KK) + 1 + size_t(4) * s.L * KK);
    hipLaunchKernelGGL(k_bww_final<T>, dim3(s.C), dim3(256), lds, stream, part, nchunk, s.C,
                       s.k, s.L, (const T*)p.w_base, (const T*)p.b_base, (const T*)p.s_base,
                       (const T*)p.w_wav, (const T*)p.s_wav, (T*)g.dw_base, (T*)g.db_base,
                       (T*)g.ds_base, (T*)g.dw_wav, (T*)g.ds_wav);
    return hipGetLastError();
}
}  // namespace

hipError_t finalize_grads(const wtconv_shape& s, const float* part, int rows, const Params& p,
                          const Grads& g, hipStream_t stream) {
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, part, rows, p, g, stream)
                                 : launch_final<__half>(s, part, rows, p, g, stream);
}

hipError_t plane_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                            const Params& p, const Grads& g, void* workspace,
                            hipStream_t stream) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    hipError_t e = prepare(v->bww, v->lds_bww);
    if (e != hipSuccess) return e;
    const int nchunk = bww_chunks(s, v->P, resident_wgs(v->bww, v->NT, v->lds_bww));
    int gpw = cdiv(cdiv(s.B, v->P), nchunk), B = s.B, C = s.C;
    float* part = static_cast<float*>(workspace);
    void* args[] = {&x, &dy, &part, &B, &C, &gpw};
    e = hipLaunchKernel(v->bww, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                        v->lds_bww, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    return finalize_grads(s, part, nchunk, p, g, stream);
}

hipError_t plane_bwd(const wtconv_shape& s, const void* x, const void* dy, const Params& p,
                     void* dx, const Grads& g, void* workspace, hipStream_t stream) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    if (!v->bwd) {
        hipError_t e = plane_apply(s, dy, p, dx, true, stream);
        if (e != hipSuccess) return e;
        return plane_bwd_weight(s, x, dy, p, g, workspace, stream);
    }
    hipError_t e = prepare(v->bwd, v->lds_bwd);
    if (e != hipSuccess) return e;
    const int nchunk = bww_chunks(s, v->P, resident_wgs(v->bwd, v->NT, v->lds_bwd));
    int gpw = cdiv(cdiv(s.B, v->P), nchunk), B = s.B, C = s.C;
    float* part = static_cast<float*>(workspace);
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    void* args[] = {&x, &dy, &wb, &sb, &ww, &sw, &dx, &part, &B, &C, &gpw};
    e = hipLaunchKernel(v->bwd, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                        v->lds_bwd, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    return finalize_grads(s, part, nchunk, p, g, stream);
}

hipError_t zero_grads(const wtconv_shape& s, const Params& p, const Grads& g,
                      hipStream_t stream) {
    return finalize_grads(s, nullptr, 0, p, g, stream);
}

}  // namespace wtc
