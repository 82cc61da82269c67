// Large planes: tile kernels for the base conv and the first LT <= 3 levels,
// deep kernels for levels LT+1..L, and the host dispatch of that path.
//
// Deep levels.  U^{LT+m}(X) = U^m(P) with P = U^LT_LL(X), the unnormalised
// 2^LT x 2^LT box sums of the plane (box sums compose), so levels LT+1..L are
// the wavelet part of the same operator applied to P, with the folded filters
// of the absolute levels.  A deep workgroup builds P of one plane in LDS,
// runs those levels there and writes, at level-LT resolution, the sum of
// their synthesized contributions; the tile kernel adds it to the level-LT LL
// coefficients (every pixel of a 2^LT block sees an LL coefficient with sign
// +1, so this is the closed-form sum of the deeper levels).  The weight
// gradient's deep levels correlate U^m(P_x) with U^m(P_dy) the same way.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_tile_variant.h"

namespace wtc {
namespace dev {

// LDS plan of a deep workgroup (floats): folded filters, then per level m of
// P (m = 0: P itself) a bordered x-side array set, then unbordered results.
struct DeepLayout {
    int hp, wp, p, LD, KK;
    __host__ __device__ int h(int m) const { return hp >> m; }
    __host__ __device__ int w(int m) const { return wp >> m; }
    __host__ __device__ int bp(int m) const { return w(m) + 2 * p; }           // bordered pitch
    __host__ __device__ int barr(int m) const { return (h(m) + 2 * p) * bp(m); }
    __host__ __device__ int nsub(int m) const { return m ? 4 : 1; }
    __host__ __device__ int wf() const { return 0; }
    __host__ __device__ int uoff(int m) const {  // bordered arrays, m = 0..LD
        int o = LD * 4 * KK;
        for (int k = 0; k < m; ++k) o += nsub(k) * barr(k);
        return o;
    }
    __host__ __device__ int coff(int m) const {  // results, m = 1..LD
        int o = uoff(LD + 1);
        for (int k = 1; k < m; ++k) o += 4 * h(k) * w(k);
        return o;
    }
    __host__ __device__ int end_apply() const { return coff(LD + 1); }
    __host__ __device__ int end_bww() const { return uoff(LD + 1) * 2 - LD * 4 * KK; }
    __host__ __device__ int u(int m, int s, int i, int j) const {
        return uoff(m) + s * barr(m) + (i + p) * bp(m) + p + j;
    }
};

// P[i][j] = sum of the 2^LT x 2^LT block of the plane -> bordered array m = 0.
template <typename T>
__device__ void box_sums(const T* __restrict__ src, int Wp, int LT, const DeepLayout& D,
                         float* lds, int base, int tid, int nt) {
    const int n = 1 << LT;
    for (int e = tid; e < D.hp * D.wp; e += nt) {
        const int i = e / D.wp, j = e % D.wp;
        const T* s = src + (size_t(i) * n) * Wp + size_t(j) * n;
        float acc = 0.f;
        for (int u = 0; u < n; ++u)
            for (int v = 0; v < n; ++v) acc += to_f(s[size_t(u) * Wp + v]);
        lds[base + (i + D.p) * D.bp(0) + D.p + j] = acc;
    }
}

// Levels m = 1..LD of P: unnormalised Haar butterflies of the LL above.
__device__ void deep_analysis(const DeepLayout& D, float* lds, int shift, int tid, int nt) {
    for (int m = 1; m <= D.LD; ++m) {
        const int h = D.h(m), w = D.w(m);
        for (int e = tid; e < h * w; e += nt) {
            const int i = e / w, j = e % w;
            const int src = D.u(m - 1, 0, 2 * i, 2 * j) + shift, sp = D.bp(m - 1);
            const float a = lds[src], b = lds[src + 1], c = lds[src + sp], d = lds[src + sp + 1];
            const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
            const int o = D.u(m, 0, i, j) + shift, A = D.barr(m);
            lds[o] = s0 + s1;
            lds[o + A] = d0 + d1;
            lds[o + 2 * A] = s0 - s1;
            lds[o + 3 * A] = d0 - d1;
        }
        __syncthreads();
    }
}

// Sum of levels LT+1..L of one plane at level-LT resolution (fp32).
template <typename T, bool FLIP>
__global__ __launch_bounds__(256) void k_deep_apply(
    const T* __restrict__ in, const T* __restrict__ ww, const T* __restrict__ sw,
    float* __restrict__ deep, int B, int C, int Hp, int Wp, int L, int LT, int K) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int b = blockIdx.x / C, c = blockIdx.x % C;
    const DeepLayout D{Hp >> LT, Wp >> LT, K / 2, L - LT, K * K};
    const int KK = D.KK;
    for (int i = tid; i < D.end_apply(); i += nt) lds[i] = 0.f;
    __syncthreads();
    // folded filters of absolute levels LT+1..L: gamma * 4^-l * K (rotated
    // for the input gradient)
    for (int i = tid; i < D.LD * 4 * KK; i += nt) {
        const int ms = i / KK, t = i % KK, m = ms / 4, s = ms % 4;
        const int la = LT + m + 1;
        const size_t gi = (size_t(la - 1) * C + c) * 4 + s;
        const int tt = FLIP ? KK - 1 - t : t;
        lds[i] = to_f(sw[gi]) * ldexpf(1.f, -2 * la) * to_f(ww[gi * KK + tt]);
    }
    box_sums<T>(in + (size_t(b) * C + c) * Hp * Wp, Wp, LT, D, lds, D.uoff(0), tid, nt);
    __syncthreads();
    deep_analysis(D, lds, 0, tid, nt);
    // subband convs
    for (int m = 1; m <= D.LD; ++m) {
        const int h = D.h(m), w = D.w(m);
        for (int e = tid; e < 4 * h * w; e += nt) {
            const int s = e / (h * w), i = (e / w) % h, j = e % w;
            const float* wk = lds + (m - 1) * 4 * KK + s * KK;
            float acc = 0.f;
            for (int uu = 0; uu < K; ++uu)
                for (int vv = 0; vv < K; ++vv)
                    acc = fmaf(wk[uu * K + vv], lds[D.u(m, s, i + uu - D.p, j + vv - D.p)], acc);
            lds[D.coff(m) + (s * h + i) * w + j] = acc;
        }
    }
    __syncthreads();
    // fold level m into the LL of level m-1, deepest first
    for (int m = D.LD; m >= 2; --m) {
        const int h = D.h(m - 1), w = D.w(m - 1), hc = D.h(m), wc = D.w(m);
        for (int e = tid; e < h * w; e += nt) {
            const int i = e / w, j = e % w;
            const float* cs = lds + D.coff(m) + (i >> 1) * wc + (j >> 1);
            const int A = hc * wc;
            const float sy = (i & 1) ? -1.f : 1.f, sx = (j & 1) ? -1.f : 1.f;
            const float e0 = fmaf(sy, cs[2 * A], cs[0]), f0 = fmaf(sy, cs[3 * A], cs[A]);
            lds[D.coff(m - 1) + i * w + j] += fmaf(sx, f0, e0);
        }
        __syncthreads();
    }
    // expand level 1 over P's grid
    {
        const int hc = D.h(1), wc = D.w(1), A = hc * wc;
        float* o = deep + (size_t(b) * C + c) * D.hp * D.wp;
        for (int e = tid; e < D.hp * D.wp; e += nt) {
            const int i = e / D.wp, j = e % D.wp;
            const float* cs = lds + D.coff(1) + (i >> 1) * wc + (j >> 1);
            const float sy = (i & 1) ? -1.f : 1.f, sx = (j & 1) ? -1.f : 1.f;
            const float e0 = fmaf(sy, cs[2 * A], cs[0]), f0 = fmaf(sy, cs[3 * A], cs[A]);
            o[e] = fmaf(sx, f0, e0);
        }
    }
}

// Correlations of levels LT+1..L of one plane, written as one full partial
// row (zeros outside those levels) at row (row0 + b) * C + c.
template <typename T>
__global__ __launch_bounds__(256) void k_deep_bww(const T* __restrict__ x,
                                                  const T* __restrict__ dy,
                                                  float* __restrict__ part, int B, int C,
                                                  int Hp, int Wp, int L, int LT, int K,
                                                  int row0, int npart) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int b = blockIdx.x / C, c = blockIdx.x % C;
    const DeepLayout D{Hp >> LT, Wp >> LT, K / 2, L - LT, K * K};
    const int KK = D.KK;
    const int shift = D.uoff(D.LD + 1) - D.uoff(0);  // dy side follows the x side
    for (int i = tid; i < D.end_bww(); i += nt) lds[i] = 0.f;
    __syncthreads();
    const size_t po = (size_t(b) * C + c) * Hp * Wp;
    box_sums<T>(x + po, Wp, LT, D, lds, D.uoff(0), tid, nt);
    box_sums<T>(dy + po, Wp, LT, D, lds, D.uoff(0) + shift, tid, nt);
    __syncthreads();
    deep_analysis(D, lds, 0, tid, nt);
    deep_analysis(D, lds, shift, tid, nt);
    float* row = part + (size_t(row0 + b) * C + c) * npart;
    for (int o = tid; o < npart; o += nt) {
        const int first = KK + 1 + LT * 4 * KK;
        float acc = 0.f;
        if (o >= first) {
            const int r = o - first, ms = r / KK, t = r % KK, m = ms / 4 + 1, s = ms % 4;
            const int uu = t / K, vv = t % K, h = D.h(m), w = D.w(m);
            for (int i = 0; i < h; ++i)
                for (int j = 0; j < w; ++j)
                    acc = fmaf(lds[D.u(m, s, i, j) + shift],
                               lds[D.u(m, s, i + uu - D.p, j + vv - D.p)], acc);
        }
        row[o] = acc;
    }
}

}  // namespace dev

namespace {
using namespace dev;

const TileVariant* find_tile(const wtconv_shape& s) {
    int n = 0;
    const TileVariant* t = nullptr;
    switch (s.k) {
        case 1: t = tile_table_k1(&n); break;
        case 3: t = tile_table_k3(&n); break;
        case 5: t = tile_table_k5(&n); break;
        case 7: t = tile_table_k7(&n); break;
        default: return nullptr;
    }
    const int LT = s.L < 3 ? s.L : 3;
    for (int i = 0; i < n; ++i)
        if (t[i].LT == LT && t[i].dtype == s.dtype) return &t[i];
    return nullptr;
}

int tile_lt(const wtconv_shape& s) { return s.L < 3 ? s.L : 3; }

DeepLayout deep_layout(const wtconv_shape& s) {
    const int LT = tile_lt(s);
    return DeepLayout{s.H >> LT, s.W >> LT, s.k / 2, s.L - LT, s.k * s.k};
}

size_t deep_apply_lds(const wtconv_shape& s) { return sizeof(float) * deep_layout(s).end_apply(); }
size_t deep_bww_lds(const wtconv_shape& s) { return sizeof(float) * deep_layout(s).end_bww(); }

constexpr size_t kMaxLds = 160 * 1024;
constexpr int kMaxTileChunks = 64;

hipError_t set_lds(const void* fn, size_t lds) {
    if (lds > 65536)
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    return hipSuccess;
}

int resident(const void* fn, int nt, size_t lds) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, nt, lds) != hipSuccess ||
        cus <= 0 || per <= 0)
        return 1024;
    return cus * per;
}

int tile_units_per_channel(const wtconv_shape& s) {
    return s.B * ((s.H + kTileH - 1) / kTileH) * ((s.W + kTileW - 1) / kTileW);
}

int tile_chunks(const wtconv_shape& s, int slots) {
    const int units = tile_units_per_channel(s);
    int want = slots / (s.C > 0 ? s.C : 1);
    if (want < 1) want = 1;
    if (want > kMaxTileChunks) want = kMaxTileChunks;
    if (want > units) want = units;
    const int upw = (units + want - 1) / want;
    return (units + upw - 1) / upw;
}

template <typename T>
const void* deep_apply_fn(bool flip) {
    return flip ? reinterpret_cast<const void*>(&k_deep_apply<T, true>)
                : reinterpret_cast<const void*>(&k_deep_apply<T, false>);
}

}  // namespace

bool tile_supported(const wtconv_shape& s) {
    const TileVariant* v = find_tile(s);
    if (!v) return false;
    // HBM items (up to 4 rows by one 16-byte vector) stay inside or outside
    // the plane
    const int vec = s.dtype == WTCONV_F32 ? 4 : 8;
    if ((s.H % 4) || (s.W % vec)) return false;
    if ((s.H % (1 << s.L)) || (s.W % (1 << s.L))) return false;
    if (s.L > tile_lt(s) && deep_bww_lds(s) > kMaxLds) return false;
    return true;
}

size_t tile_workspace_bytes(const wtconv_shape& s) {
    if (!tile_supported(s) || s.B == 0 || s.C == 0) return 0;
    const int LT = tile_lt(s);
    const size_t KK = size_t(s.k) * s.k, npart = KK + 1 + 4 * size_t(s.L) * KK;
    const int units = tile_units_per_channel(s);
    const size_t chunks = size_t(units < kMaxTileChunks ? units : kMaxTileChunks) +
                          (s.L > LT ? size_t(s.B) : 0);
    const size_t bww = chunks * s.C * npart * sizeof(float);
    const size_t deep =
        s.L > LT ? size_t(s.B) * s.C * (s.H >> LT) * (s.W >> LT) * sizeof(float) : 0;
    return bww > deep ? bww : deep;
}

hipError_t tile_apply(const wtconv_shape& s, const void* in, const Params& p, void* out,
                      bool flip, void* workspace, hipStream_t stream) {
    const TileVariant* v = find_tile(s);
    if (!v) return hipErrorInvalidValue;
    const int LT = tile_lt(s);
    int B = s.B, C = s.C, H = s.H, W = s.W, L = s.L, K = s.k, LTv = LT;
    float* deep = nullptr;
    hipError_t e;
    if (s.L > LT) {
        deep = static_cast<float*>(workspace);
        const void* fn = s.dtype == WTCONV_F32 ? deep_apply_fn<float>(flip)
                                               : deep_apply_fn<__half>(flip);
        const size_t lds = deep_apply_lds(s);
        if ((e = set_lds(fn, lds)) != hipSuccess) return e;
        const void* ww = p.w_wav;
        const void* sw = p.s_wav;
        void* args[] = {&in, &ww, &sw, &deep, &B, &C, &H, &W, &L, &LTv, &K};
        e = hipLaunchKernel(fn, dim3(unsigned(B) * unsigned(C)), dim3(256), args, lds, stream);
        if (e != hipSuccess) return e;
    }
    const void* fn = flip ? v->bwi : v->fwd;
    if ((e = set_lds(fn, v->lds_apply)) != hipSuccess) return e;
    const long total = long(s.C) * tile_units_per_channel(s);
    long nwg = resident(fn, v->NT, v->lds_apply);
    if (nwg > total) nwg = total;
    const void* bb = flip ? p.w_base : p.b_base;  // unread when flipped
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    const float* dp = deep;
    void* args[] = {&in, &wb, &bb, &sb, &ww, &sw, &dp, &out, &B, &C, &H, &W};
    e = hipLaunchKernel(fn, dim3(unsigned(nwg)), dim3(v->NT), args, v->lds_apply, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t tile_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                           const Params& p, const Grads& g, void* workspace,
                           hipStream_t stream) {
    const TileVariant* v = find_tile(s);
    if (!v) return hipErrorInvalidValue;
    const int LT = tile_lt(s);
    hipError_t e;
    if ((e = set_lds(v->bww, v->lds_bww)) != hipSuccess) return e;
    const int nchunk = tile_chunks(s, resident(v->bww, v->NT, v->lds_bww));
    const int units = tile_units_per_channel(s);
    int upw = (units + nchunk - 1) / nchunk;
    int B = s.B, C = s.C, H = s.H, W = s.W, L = s.L, K = s.k, LTv = LT;
    int npart = s.k * s.k * (1 + 4 * s.L) + 1;
    float* part = static_cast<float*>(workspace);
    {
        void* args[] = {&x, &dy, &part, &B, &C, &H, &W, &upw, &npart};
        e = hipLaunchKernel(v->bww, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                            v->lds_bww, stream);
        if (e != hipSuccess) return e;
    }
    int rows = nchunk;
    if (s.L > LT) {
        const void* fn = s.dtype == WTCONV_F32
                             ? reinterpret_cast<const void*>(&k_deep_bww<float>)
                             : reinterpret_cast<const void*>(&k_deep_bww<__half>);
        const size_t lds = deep_bww_lds(s);
        if ((e = set_lds(fn, lds)) != hipSuccess) return e;
        int row0 = nchunk;
        void* args[] = {&x, &dy, &part, &B, &C, &H, &W, &L, &LTv, &K, &row0, &npart};
        e = hipLaunchKernel(fn, dim3(unsigned(B) * unsigned(C)), dim3(256), args, lds, stream);
        if (e != hipSuccess) return e;
        rows += s.B;
    }
    return finalize_grads(s, part, rows, p, g, stream);
}

}  // namespace wtc
