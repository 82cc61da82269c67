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

// Outputs per work item along a row of a deep conv, and row chunks per
// (level, subband, tap row) of a deep correlation.
constexpr int kDeepRS = 8, kDeepNCH = 12;
// Threads of a deep workgroup (one per plane).  A deep workgroup is a chain
// of short phases over one plane's box sums; 512 threads split its
// correlations into twice the row chunks of 256 (512², L = 5: k_deep_bww
// 53 -> ~41 us, the fused backward 1008 -> 990 us; 1024 threads gain no
// more).
constexpr int kDeepNT = 512;

// LDS plan of a deep workgroup (floats): folded filters, then per level
// m = 1..LD of P a bordered x-side array set (P itself, level 0, is read
// from device memory straight into level 1's butterflies and never stored),
// then unbordered results.
// Rows are padded to whole kDeepRS segments so that a segment's window stays
// in its row.  Both pitches are odd: the lanes of a half-wavefront take
// consecutive rows (and segments of kDeepRS columns), which an odd pitch
// puts on distinct banks; an even one folds them onto a few (with pitch 36,
// eight rows on eight banks: every window read 8-way conflicted).
struct DeepLayout {
    int hp, wp, p, LD, KK;
    __host__ __device__ int h(int m) const { return hp >> m; }
    __host__ __device__ int w(int m) const { return wp >> m; }
    __host__ __device__ int bp(int m) const {  // bordered pitch
        return ((w(m) + kDeepRS - 1) / kDeepRS * kDeepRS + 2 * p) | 1;
    }
    __host__ __device__ int rp(int m) const { return w(m) | 1; }  // result pitch
    __host__ __device__ int barr(int m) const { return (h(m) + 2 * p) * bp(m); }
    __host__ __device__ int nsub(int m) const { return m ? 4 : 1; }
    __host__ __device__ int wf() const { return 0; }
    __host__ __device__ int uoff(int m) const {  // bordered arrays, m = 1..LD
        int o = LD * 4 * KK;
        for (int k = 1; k < m; ++k) o += nsub(k) * barr(k);
        return o;
    }
    __host__ __device__ int coff(int m) const {  // results, m = 1..LD
        int o = uoff(LD + 1);
        for (int k = 1; k < m; ++k) o += 4 * h(k) * rp(k);
        return o;
    }
    __host__ __device__ int end_apply() const { return coff(LD + 1); }
    __host__ __device__ int end_bww() const { return uoff(LD + 1) * 2 - LD * 4 * KK; }
    // the dy side of the weight-gradient kernel follows the x side
    __host__ __device__ int dy_shift() const { return uoff(LD + 1) - uoff(1); }
    // correlation partials after the two array sets: [item][K]
    __host__ __device__ int end_bww_red(int K) const {
        return end_bww() + LD * 4 * K * kDeepNCH * K;
    }
    __host__ __device__ int u(int m, int s, int i, int j) const {
        return uoff(m) + s * barr(m) + (i + p) * bp(m) + p + j;
    }
};

// e / d and e % d for 0 <= e < 2^22 and d >= 1, from d's fp32 reciprocal.
// The two roundings (reciprocal, product) are each within 2^-23 relative,
// so on a quotient below 2^22 the truncated product is off by at most one,
// which the remainder's sign corrects.  The deep phases index an element
// per item; the integer division this replaces cost them more VALU issue
// than the arithmetic on the element.
struct DivMod {
    int d;
    float r;
    __device__ explicit DivMod(int d_) : d(d_), r(1.f / float(d_)) {}
    __device__ int2 operator()(int e) const {
        int q = int(float(e) * r), m = e - q * d;
        if (m < 0) {
            --q;
            m += d;
        } else if (m >= d) {
            ++q;
            m -= d;
        }
        return make_int2(q, m);
    }
};

// n floats from a (16-byte aligned) set to zero, 16 bytes per store.
__device__ void zero_lds(float* a, int n, int tid, int nt) {
    const int n4 = n >> 2;
    float4* a4 = reinterpret_cast<float4*>(a);
    for (int i = tid; i < n4; i += nt) a4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 4 * n4 + tid; i < n; i += nt) a[i] = 0.f;
}

// Four elements at src, as float, read with the non-temporal hint: the box
// sums stream their tensor once, and reading it so leaves the caches to
// the tile kernels around them (512², L = 5: forward 483 -> 472 us, fused
// backward 913 -> 897 us, one box-sum pass each).
template <typename T>
__device__ __forceinline__ void load4_nt(const T* __restrict__ src, float (&v)[4]) {
    if constexpr (std::is_same<T, float>::value) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 q = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src));
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        const u2 q = __builtin_nontemporal_load(reinterpret_cast<const u2*>(src));
        union { unsigned int u[2]; __half2 h[2]; } pk;
        pk.u[0] = q.x;
        pk.u[1] = q.y;
        const float2 fa = __half22float2(pk.h[0]), fb = __half22float2(pk.h[1]);
        v[0] = fa.x; v[1] = fa.y; v[2] = fb.x; v[3] = fb.y;
    }
}

// P = U^LT_LL of every plane: P[i][j] is the sum of the plane's 2^LT x 2^LT
// block (i, j).  One workgroup per row of P; each lane sums a 4-column strip
// of the block rows with one vector load per row, then the n/4 lanes of a
// block add their strips with cross-lane exchanges (n = 2^LT >= 4).
template <typename T>
__global__ __launch_bounds__(128) void k_box_sums(const T* __restrict__ src,
                                                  float* __restrict__ P, int Hp, int Wp,
                                                  int LT) {
    const int n = 1 << LT, hd = Hp >> LT, wd = Wp >> LT;
    const int row = blockIdx.x % hd;
    const size_t plane = blockIdx.x / hd;
    const T* s0 = src + (plane * Hp + size_t(row) * n) * Wp;
    float* out = P + (plane * hd + row) * wd;
    const int nq = Wp / 4, per = n / 4;  // quads per row, quads per block
    for (int q0 = 0; q0 < nq; q0 += blockDim.x) {
        const int q = q0 + threadIdx.x;
        float acc = 0.f;
        if (q < nq && n == 8) {
            // the blocks of three tile levels: all eight row loads in flight
            // at once, then the sums in the same order as below
            float v[8][4];
#pragma unroll
            for (int r = 0; r < 8; ++r) load4_nt<T>(s0 + size_t(r) * Wp + 4 * q, v[r]);
#pragma unroll
            for (int r = 0; r < 8; ++r) acc += (v[r][0] + v[r][1]) + (v[r][2] + v[r][3]);
        } else if (q < nq) {
            for (int r = 0; r < n; ++r) {
                float v[4];
                load4_nt<T>(s0 + size_t(r) * Wp + 4 * q, v);
                acc += (v[0] + v[1]) + (v[2] + v[3]);
            }
        }
        // lanes q, q^1, ... of one block are in one wavefront and either all
        // hold a quad or none does (nq is a multiple of per)
        for (int k = 1; k < per; k <<= 1) acc += __shfl_xor(acc, k);
        if (q < nq && (q % per) == 0) out[q / per] = acc;
    }
}

// Level 1 of one plane from its box sums P in device memory: each item
// loads a 2 x 2 block of P (two 8-byte loads; P's width is even) and writes
// its four unnormalised Haar coefficients.  Four items' loads are issued
// before their butterflies, so a lane waits on one device-memory round trip
// per four items, not per item.
__device__ void load_level1(const float* __restrict__ Pp, const DeepLayout& D, float* lds,
                            int shift, int tid, int nt) {
    constexpr int U = 4;
    const int h = D.h(1), w = D.w(1), n = h * w, A = D.barr(1), wp = D.wp;
    const int base = D.u(1, 0, 0, 0) + shift, bp = D.bp(1);
    const DivMod by_w(w);
    for (int e0 = tid; e0 < n; e0 += U * nt) {
        float2 top[U], bot[U];
        int2 ij[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ij[u] = by_w(min(e0 + u * nt, n - 1));
            const float* q = Pp + size_t(2 * ij[u].x) * wp + 2 * ij[u].y;
            top[u] = *reinterpret_cast<const float2*>(q);
            bot[u] = *reinterpret_cast<const float2*>(q + wp);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (e0 + u * nt >= n) break;
            const float s0 = top[u].x + top[u].y, d0 = top[u].x - top[u].y;
            const float s1 = bot[u].x + bot[u].y, d1 = bot[u].x - bot[u].y;
            const int o = base + ij[u].x * bp + ij[u].y;
            lds[o] = s0 + s1;
            lds[o + A] = d0 + d1;
            lds[o + 2 * A] = s0 - s1;
            lds[o + 3 * A] = d0 - d1;
        }
    }
}

// Levels m = 2..LD of P: unnormalised Haar butterflies of the LL above.
__device__ void deep_analysis(const DeepLayout& D, float* lds, int shift, int tid, int nt) {
    for (int m = 2; m <= D.LD; ++m) {
        const int h = D.h(m), w = D.w(m), sp = D.bp(m - 1), dp = D.bp(m), A = D.barr(m);
        const int sb = D.u(m - 1, 0, 0, 0) + shift, db = D.u(m, 0, 0, 0) + shift;
        const DivMod by_w(w);
        for (int e = tid; e < h * w; e += nt) {
            const int2 ij = by_w(e);
            const int src = sb + 2 * ij.x * sp + 2 * ij.y;
            const float a = lds[src], b = lds[src + 1], c = lds[src + sp], d = lds[src + sp + 1];
            const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
            const int o = db + ij.x * dp + ij.y;
            lds[o] = s0 + s1;
            lds[o + A] = d0 + d1;
            lds[o + 2 * A] = s0 - s1;
            lds[o + 3 * A] = d0 - d1;
        }
        __syncthreads();
    }
}

// Sum of levels LT+1..L of one plane at level-LT resolution (fp32), from
// the plane's box sums P.  Each work item computes kDeepRS outputs of one
// row of one subband from a K x (kDeepRS + K - 1) window held in registers.
template <typename T, int K, bool FLIP>
__global__ __launch_bounds__(kDeepNT) void k_deep_apply(
    const float* __restrict__ P, const T* __restrict__ ww, const T* __restrict__ sw,
    float* __restrict__ deep, int B, int C, int Hp, int Wp, int L, int LT) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int b = blockIdx.x / C, c = blockIdx.x % C;
    constexpr int KK = K * K, RS = kDeepRS;
    const DeepLayout D{Hp >> LT, Wp >> LT, K / 2, L - LT, KK};
    // the bordered arrays start at zero: their borders and the row padding
    // past a level's width are the convs' zero padding (the interiors, and
    // every result read later, are written below)
    zero_lds(lds + D.uoff(1), D.uoff(D.LD + 1) - D.uoff(1), tid, nt);
    // folded filters of absolute levels LT+1..L, below the bordered arrays:
    // gamma * 4^-l * K (rotated for the input gradient)
    for (int i = tid; i < D.LD * 4 * KK; i += nt) {
        const int ms = i / KK, t = i % KK, m = ms / 4, s = ms % 4;
        const int la = LT + m + 1;
        const size_t gi = (size_t(la - 1) * C + c) * 4 + s;
        const int tt = FLIP ? KK - 1 - t : t;
        lds[i] = to_f(sw[gi]) * ldexpf(1.f, -2 * la) * to_f(ww[gi * KK + tt]);
    }
    __syncthreads();
    load_level1(P + (size_t(b) * C + c) * D.hp * D.wp, D, lds, 0, tid, nt);
    __syncthreads();
    deep_analysis(D, lds, 0, tid, nt);
    // subband convs
    for (int m = 1; m <= D.LD; ++m) {
        const int h = D.h(m), w = D.w(m), nseg = (w + RS - 1) / RS;
        const int bpm = D.bp(m), A = D.barr(m), um = D.uoff(m), rpm = D.rp(m), cm = D.coff(m);
        const DivMod by_seg(nseg), by_h(h);
        for (int e = tid; e < 4 * h * nseg; e += nt) {
            const int2 rs = by_seg(e), si = by_h(rs.x);  // rs.x = s * h + i
            const int s = si.x, i = si.y, j0 = rs.y * RS;
            const float* wk = lds + (m - 1) * 4 * KK + s * KK;
            float acc[RS];
#pragma unroll
            for (int r = 0; r < RS; ++r) acc[r] = 0.f;
#pragma unroll
            for (int uu = 0; uu < K; ++uu) {
                // row i + uu - p from column j0 - p of the bordered array
                const float* src = lds + um + s * A + (i + uu) * bpm + j0;
                float row[RS + K - 1];
#pragma unroll
                for (int t = 0; t < RS + K - 1; ++t) row[t] = src[t];
#pragma unroll
                for (int vv = 0; vv < K; ++vv) {
                    const float wv = wk[uu * K + vv];
#pragma unroll
                    for (int r = 0; r < RS; ++r) acc[r] = fmaf(wv, row[r + vv], acc[r]);
                }
            }
            float* o = lds + cm + rs.x * rpm + j0;
#pragma unroll
            for (int r = 0; r < RS; ++r)
                if (j0 + r < w) o[r] = acc[r];
        }
    }
    __syncthreads();
    // fold level m into the LL of level m-1, deepest first
    // (one item per coarse position: its four subbands give the 2 x 2 fine
    // block, (LL + sy HL) + sx (LH + sy HH) with sy, sx = -1 on odd rows,
    // columns; levels halve exactly, the plane being a multiple of 2^L)
    for (int m = D.LD; m >= 2; --m) {
        const int hc = D.h(m), wc = D.w(m), rc = D.rp(m), A = hc * rc, rf = D.rp(m - 1);
        const float* cm = lds + D.coff(m);
        float* fm = lds + D.coff(m - 1);
        const DivMod by_w(wc);
        for (int e = tid; e < hc * wc; e += nt) {
            const int2 ij = by_w(e);
            const float* cs = cm + ij.x * rc + ij.y;
            const float ll = cs[0], lh = cs[A], hl = cs[2 * A], hh = cs[3 * A];
            const float e0 = ll + hl, f0 = lh + hh, e1 = ll - hl, f1 = lh - hh;
            float* f = fm + 2 * ij.x * rf + 2 * ij.y;
            f[0] += e0 + f0;
            f[1] += e0 - f0;
            f[rf] += e1 + f1;
            f[rf + 1] += e1 - f1;
        }
        __syncthreads();
    }
    // expand level 1 over P's grid
    // (the same 2 x 2 blocks, two 8-byte stores each: P's width is even)
    {
        const int hc = D.h(1), wc = D.w(1), rc = D.rp(1), A = hc * rc, wp = D.wp;
        const float* cm = lds + D.coff(1);
        float* o = deep + (size_t(b) * C + c) * D.hp * wp;
        const DivMod by_w(wc);
        for (int e = tid; e < hc * wc; e += nt) {
            const int2 ij = by_w(e);
            const float* cs = cm + ij.x * rc + ij.y;
            const float ll = cs[0], lh = cs[A], hl = cs[2 * A], hh = cs[3 * A];
            const float e0 = ll + hl, f0 = lh + hh, e1 = ll - hl, f1 = lh - hh;
            float* q = o + size_t(2 * ij.x) * wp + 2 * ij.y;
            *reinterpret_cast<float2*>(q) = make_float2(e0 + f0, e0 - f0);
            *reinterpret_cast<float2*>(q + wp) = make_float2(e1 + f1, e1 - f1);
        }
    }
}

// Correlations of levels LT+1..L of one plane (from the box sums of x and
// dy), written as one full partial row (zeros outside those levels) at row
// (row0 + b) * C + c.  A work item is one (level, subband, tap row) over a
// chunk of the rows, with K tap accumulators; the chunks are summed in order.
template <int K>
__global__ __launch_bounds__(kDeepNT) void k_deep_bww(const float* __restrict__ px,
                                                  const float* __restrict__ pdy,
                                                  float* __restrict__ part, int B, int C,
                                                  int Hp, int Wp, int L, int LT, int row0,
                                                  int npart) {
    extern __shared__ float lds[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int b = blockIdx.x / C, c = blockIdx.x % C;
    constexpr int KK = K * K, NCH = kDeepNCH;
    const DeepLayout D{Hp >> LT, Wp >> LT, K / 2, L - LT, KK};
    const int shift = D.dy_shift();
    // both bordered array sets (x's, then dy's) start at zero
    zero_lds(lds + D.uoff(1), D.end_bww() - D.uoff(1), tid, nt);
    __syncthreads();
    const size_t po = (size_t(b) * C + c) * D.hp * D.wp;
    load_level1(px + po, D, lds, 0, tid, nt);
    load_level1(pdy + po, D, lds, shift, tid, nt);
    __syncthreads();
    deep_analysis(D, lds, 0, tid, nt);
    deep_analysis(D, lds, shift, tid, nt);
    float* red = lds + D.end_bww();
    const int items = D.LD * 4 * K * NCH;
    for (int e = tid; e < items; e += nt) {
        const int ch = e % NCH;
        int r = e / NCH;
        const int uu = r % K;
        r /= K;
        const int s = r % 4, m = r / 4 + 1;
        const int h = D.h(m), w = D.w(m);
        const int i0 = ch * h / NCH, i1 = (ch + 1) * h / NCH;
        float acc[K];
#pragma unroll
        for (int vv = 0; vv < K; ++vv) acc[vv] = 0.f;
        // kDeepRS columns per step from a register window (rows are padded
        // to whole kDeepRS segments, with zeros past the level's width):
        // kDeepRS + (kDeepRS + K - 1) LDS reads per kDeepRS * K FMAs
        constexpr int RS = kDeepRS;
        for (int i = i0; i < i1; ++i)
            for (int j0 = 0; j0 < w; j0 += RS) {
                const float* vr = lds + D.u(m, s, i, j0) + shift;
                const float* xr = lds + D.u(m, s, i + uu - D.p, j0 - D.p);
                float dv[RS], xw[RS + K - 1];
#pragma unroll
                for (int r = 0; r < RS; ++r) dv[r] = vr[r];
#pragma unroll
                for (int r = 0; r < RS + K - 1; ++r) xw[r] = xr[r];
#pragma unroll
                for (int r = 0; r < RS; ++r)
#pragma unroll
                    for (int vv = 0; vv < K; ++vv) acc[vv] = fmaf(dv[r], xw[r + vv], acc[vv]);
            }
#pragma unroll
        for (int vv = 0; vv < K; ++vv) red[e * K + vv] = acc[vv];
    }
    __syncthreads();
    float* row = part + (size_t(row0 + b) * C + c) * npart;
    const int first = KK + 1 + LT * 4 * KK;
    for (int o = tid; o < npart; o += nt) {
        float acc = 0.f;
        if (o >= first) {
            const int r = o - first, ms = r / KK, t = r % KK;
            const int uu = t / K, vv = t % K;
            const int e0 = (ms * K + uu) * NCH;  // ms = (m - 1) * 4 + s
            for (int ch = 0; ch < NCH; ++ch) acc += red[(e0 + ch) * K + vv];
        }
        row[o] = acc;
    }
}

// Deep levels of planes whose box sums do not fit one workgroup's LDS: the
// same arithmetic as k_deep_apply / k_deep_bww, staged through device memory
// one level at a time (the box sums are 1/4^LT of the input, so these passes
// are small next to the tiles).  Level m of every plane is one array
// [plane][subband][h(m)][w(m)] of fp32.
struct DeepGlobal {
    int planes, hp, wp, LD;
    __host__ __device__ int h(int m) const { return hp >> m; }
    __host__ __device__ int w(int m) const { return wp >> m; }
    __host__ __device__ size_t level_size(int m) const { return size_t(4) * planes * h(m) * w(m); }
    __host__ __device__ size_t level_off(int m) const {  // floats, m = 1..LD + 1
        size_t o = 0;
        for (int k = 1; k < m; ++k) o += level_size(k);
        return o;
    }
};

// One unnormalised Haar level of every plane: the 2 x 2 blocks of the source
// LL (plane stride `sps`, row pitch `sp`) into the four subbands of `dst`.
__global__ __launch_bounds__(256) void k_gdeep_analysis(const float* __restrict__ src,
                                                        size_t sps, int sp,
                                                        float* __restrict__ dst, int planes,
                                                        int h, int w) {
    const size_t n = size_t(planes) * h * w, A = size_t(h) * w;
    for (size_t e = size_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += size_t(gridDim.x) * blockDim.x) {
        const int j = int(e % w);
        const size_t r = e / w;
        const int i = int(r % h);
        const size_t pl = r / h;
        const float* s0 = src + pl * sps + size_t(2 * i) * sp + 2 * j;
        const float a = s0[0], b = s0[1], c = s0[sp], d = s0[sp + 1];
        const float x0 = a + b, d0 = a - b, x1 = c + d, d1 = c - d;
        float* o = dst + pl * 4 * A + size_t(i) * w + j;
        o[0] = x0 + x1;
        o[A] = d0 + d1;
        o[2 * A] = x0 - x1;
        o[3 * A] = d0 - d1;
    }
}

// Folded-filter conv of one (plane, subband) of absolute level `la` per
// workgroup, 'same' zero padding, taps in the order of k_deep_apply.
template <typename T, int K, bool FLIP>
__global__ __launch_bounds__(256) void k_gdeep_conv(const float* __restrict__ U,
                                                    float* __restrict__ out,
                                                    const T* __restrict__ ww,
                                                    const T* __restrict__ sw, int C, int h,
                                                    int w, int la) {
    constexpr int KK = K * K, p = K / 2;
    __shared__ float wk[KK];
    const int ps = blockIdx.x, s = ps % 4, c = (ps / 4) % C;
    if (threadIdx.x < KK) {
        const int t = threadIdx.x, tt = FLIP ? KK - 1 - t : t;
        const size_t gi = (size_t(la - 1) * C + c) * 4 + s;
        wk[t] = to_f(sw[gi]) * ldexpf(1.f, -2 * la) * to_f(ww[gi * KK + tt]);
    }
    __syncthreads();
    const float* u = U + size_t(ps) * h * w;
    float* o = out + size_t(ps) * h * w;
    for (int e = threadIdx.x; e < h * w; e += blockDim.x) {
        const int i = e / w, j = e % w;
        float acc = 0.f;
#pragma unroll
        for (int uu = 0; uu < K; ++uu) {
            const int y = i + uu - p;
            if (y < 0 || y >= h) continue;
#pragma unroll
            for (int vv = 0; vv < K; ++vv) {
                const int x = j + vv - p;
                if (x >= 0 && x < w) acc = fmaf(wk[uu * K + vv], u[y * w + x], acc);
            }
        }
        o[e] = acc;
    }
}

// The same conv with the (plane, subband) staged in LDS first: a bordered
// array (zero borders of p, rows padded to whole kDeepRS segments, odd
// pitch), then kDeepRS outputs of a row per item from a register window, as
// in k_deep_apply.  The taps and their order are k_gdeep_conv's (taps past
// the level read the border's zeros instead of being skipped).  Device
// memory is read once per element, coalesced, instead of once per tap with
// a bounds test.  LDS: K^2 filters + (h + 2p) * pitch floats, for levels
// where that fits 64 KB (gdeep_conv_lds_bytes).
template <typename T, int K, bool FLIP>
__global__ __launch_bounds__(256) void k_gdeep_conv_lds(const float* __restrict__ U,
                                                        float* __restrict__ out,
                                                        const T* __restrict__ ww,
                                                        const T* __restrict__ sw, int C, int h,
                                                        int w, int la) {
    constexpr int KK = K * K, p = K / 2, RS = kDeepRS;
    extern __shared__ float lds[];
    const int ps = blockIdx.x, s = ps % 4, c = (ps / 4) % C;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int nseg = (w + RS - 1) / RS, bp = (nseg * RS + 2 * p) | 1, rows = h + 2 * p;
    float* wk = lds;
    float* a = lds + KK;
    if (tid < KK) {
        const int tt = FLIP ? KK - 1 - tid : tid;
        const size_t gi = (size_t(la - 1) * C + c) * 4 + s;
        wk[tid] = to_f(sw[gi]) * ldexpf(1.f, -2 * la) * to_f(ww[gi * KK + tt]);
    }
    const float* u = U + size_t(ps) * h * w;
    const DivMod by_bp(bp);
    for (int e = tid; e < rows * bp; e += nt) {
        const int2 rj = by_bp(e);
        const int y = rj.x - p, x = rj.y - p;
        a[e] = y >= 0 && y < h && x >= 0 && x < w ? u[y * w + x] : 0.f;
    }
    __syncthreads();
    float* o = out + size_t(ps) * h * w;
    const DivMod by_seg(nseg);
    for (int e = tid; e < h * nseg; e += nt) {
        const int2 is = by_seg(e);
        const int i = is.x, j0 = is.y * RS;
        float acc[RS];
#pragma unroll
        for (int r = 0; r < RS; ++r) acc[r] = 0.f;
#pragma unroll
        for (int uu = 0; uu < K; ++uu) {
            // row i + uu - p of the level from column j0 - p, bordered
            const float* src = a + (i + uu) * bp + j0;
            float row[RS + K - 1];
#pragma unroll
            for (int t = 0; t < RS + K - 1; ++t) row[t] = src[t];
#pragma unroll
            for (int vv = 0; vv < K; ++vv) {
                const float wv = wk[uu * K + vv];
#pragma unroll
                for (int r = 0; r < RS; ++r) acc[r] = fmaf(wv, row[r + vv], acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < RS; ++r)
            if (j0 + r < w) o[i * w + j0 + r] = acc[r];
    }
}

// The conv outputs of one level synthesised one level down, with the signs
// of k_deep_apply: added to the next finer LL (`accumulate`), or written as
// the level-LT contribution D.
__global__ __launch_bounds__(256) void k_gdeep_synth(const float* __restrict__ cm, int hc,
                                                     int wc, float* __restrict__ dst,
                                                     size_t dps, int dp, int planes,
                                                     bool accumulate) {
    const int h = 2 * hc, w = 2 * wc;
    const size_t n = size_t(planes) * h * w, A = size_t(hc) * wc;
    for (size_t e = size_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += size_t(gridDim.x) * blockDim.x) {
        const int j = int(e % w);
        const size_t r = e / w;
        const int i = int(r % h);
        const size_t pl = r / h;
        const float* cs = cm + pl * 4 * A + size_t(i >> 1) * wc + (j >> 1);
        const float sy = (i & 1) ? -1.f : 1.f, sx = (j & 1) ? -1.f : 1.f;
        const float e0 = fmaf(sy, cs[2 * A], cs[0]), f0 = fmaf(sy, cs[3 * A], cs[A]);
        const float v = fmaf(sx, f0, e0);
        float* d = dst + pl * dps + size_t(i) * dp + j;
        *d = accumulate ? *d + v : v;
    }
}

// Correlation taps of one (plane, level, subband) per workgroup: V (dy side)
// against the shifted U (x side), each lane over a strided share of the
// positions, then summed over the lanes in order into the plane's partial
// row (row0 + b) * C + c.  The workgroup of the first subband of the first
// level also zeroes the row's slots below the deep levels.
template <int K>
__global__ __launch_bounds__(256) void k_gdeep_corr(const float* __restrict__ ux,
                                                    const float* __restrict__ vdy,
                                                    DeepGlobal G, float* __restrict__ part,
                                                    int C, int LT, int row0, int npart) {
    constexpr int KK = K * K, p = K / 2, NT = 256;
    __shared__ float red[NT * KK];
    const int tid = threadIdx.x;
    const int ms = blockIdx.x % (G.LD * 4), pl = blockIdx.x / (G.LD * 4);
    const int m = ms / 4 + 1, s = ms % 4, h = G.h(m), w = G.w(m);
    const size_t off = G.level_off(m) + (size_t(pl) * 4 + s) * h * w;
    const float* u = ux + off;
    const float* v = vdy + off;
    float acc[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[t] = 0.f;
    // a thread takes RS columns of a row per item: RS values of dy's level
    // and, per tap row, RS + K - 1 of x's (masked at the level's edges), so
    // RS * KK FMAs per RS + K (RS + K - 1) loads instead of KK + 1 per KK
    constexpr int RS = 8;
    const int nb = (w + RS - 1) / RS;
    for (int e = tid; e < h * nb; e += NT) {
        const int i = e / nb, j0 = (e % nb) * RS;
        float dv[RS];
#pragma unroll
        for (int r = 0; r < RS; ++r) dv[r] = j0 + r < w ? v[i * w + j0 + r] : 0.f;
#pragma unroll
        for (int uu = 0; uu < K; ++uu) {
            const int y = i + uu - p;
            if (y < 0 || y >= h) continue;
            float xw[RS + K - 1];
#pragma unroll
            for (int r = 0; r < RS + K - 1; ++r) {
                const int x = j0 + r - p;
                xw[r] = x >= 0 && x < w ? u[y * w + x] : 0.f;
            }
#pragma unroll
            for (int r = 0; r < RS; ++r)
#pragma unroll
                for (int vv = 0; vv < K; ++vv)
                    acc[uu * K + vv] = fmaf(dv[r], xw[r + vv], acc[uu * K + vv]);
        }
    }
#pragma unroll
    for (int t = 0; t < KK; ++t) red[tid * KK + t] = acc[t];
    __syncthreads();
    const int b = pl / C, c = pl % C;
    float* row = part + (size_t(row0 + b) * C + c) * npart;
    const int first = KK + 1 + LT * 4 * KK;
    for (int t = tid; t < KK; t += NT) {
        float sum = 0.f;
        for (int q = 0; q < NT; ++q) sum += red[q * KK + t];
        row[first + ms * KK + t] = sum;
    }
    if (ms == 0)
        for (int o = tid; o < first; o += NT) row[o] = 0.f;
}

// The same taps with the (plane, level, subband) staged in LDS: U bordered
// (zero borders of p, rows padded to whole kDeepRS segments, odd pitch), V
// padded with zeros to whole segments.  A work item is one tap row over a
// chunk of the rows (K accumulators, kDeepRS columns per step from register
// windows, as in k_deep_bww); the chunks are summed in order.  Gathered
// from device memory with a bounds test per element, and summed over the
// 256 lanes one by one, the taps had cost ~250 us per 1024² step.  LDS:
// gdeep_corr_lds_bytes, sized for level 1, the largest.
template <int K>
__global__ __launch_bounds__(256) void k_gdeep_corr_lds(const float* __restrict__ ux,
                                                        const float* __restrict__ vdy,
                                                        DeepGlobal G, float* __restrict__ part,
                                                        int C, int LT, int row0, int npart) {
    constexpr int KK = K * K, p = K / 2, RS = kDeepRS, NCH = 256 / K;
    extern __shared__ float lds[];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int ms = blockIdx.x % (G.LD * 4), pl = blockIdx.x / (G.LD * 4);
    const int m = ms / 4 + 1, s = ms % 4, h = G.h(m), w = G.w(m);
    const size_t off = G.level_off(m) + (size_t(pl) * 4 + s) * h * w;
    const int nseg = (w + RS - 1) / RS, bpu = (nseg * RS + 2 * p) | 1, bpv = (nseg * RS) | 1;
    const int nu = (h + 2 * p) * bpu, nv = h * bpv;
    float* a = lds;       // U, bordered
    float* v = a + nu;    // V, padded
    float* red = v + nv;  // [item][K]
    const DivMod by_bpu(bpu), by_bpv(bpv);
    for (int e = tid; e < nu; e += nt) {
        const int2 rj = by_bpu(e);
        const int y = rj.x - p, x = rj.y - p;
        a[e] = y >= 0 && y < h && x >= 0 && x < w ? ux[off + size_t(y) * w + x] : 0.f;
    }
    for (int e = tid; e < nv; e += nt) {
        const int2 rj = by_bpv(e);
        v[e] = rj.y < w ? vdy[off + size_t(rj.x) * w + rj.y] : 0.f;
    }
    __syncthreads();
    if (tid < K * NCH) {
        const int uu = tid / NCH, ch = tid % NCH;
        const int i0 = ch * h / NCH, i1 = (ch + 1) * h / NCH;
        float acc[K];
#pragma unroll
        for (int vv = 0; vv < K; ++vv) acc[vv] = 0.f;
        for (int i = i0; i < i1; ++i)
            for (int j0 = 0; j0 < nseg * RS; j0 += RS) {
                const float* vr = v + i * bpv + j0;
                // row i + uu - p of U from column j0 - p, bordered
                const float* xr = a + (i + uu) * bpu + j0;
                float dv[RS], xw[RS + K - 1];
#pragma unroll
                for (int r = 0; r < RS; ++r) dv[r] = vr[r];
#pragma unroll
                for (int r = 0; r < RS + K - 1; ++r) xw[r] = xr[r];
#pragma unroll
                for (int r = 0; r < RS; ++r)
#pragma unroll
                    for (int vv = 0; vv < K; ++vv) acc[vv] = fmaf(dv[r], xw[r + vv], acc[vv]);
            }
#pragma unroll
        for (int vv = 0; vv < K; ++vv) red[tid * K + vv] = acc[vv];
    }
    __syncthreads();
    const int b = pl / C, c = pl % C;
    float* row = part + (size_t(row0 + b) * C + c) * npart;
    const int first = KK + 1 + LT * 4 * KK;
    for (int t = tid; t < KK; t += nt) {
        const int uu = t / K, vv = t % K;
        float sum = 0.f;
        for (int ch = 0; ch < NCH; ++ch) sum += red[(uu * NCH + ch) * K + vv];
        row[first + ms * KK + t] = sum;
    }
    if (ms == 0)
        for (int o = tid; o < first; o += nt) row[o] = 0.f;
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
size_t deep_bww_lds(const wtconv_shape& s) {
    return sizeof(float) * deep_layout(s).end_bww_red(s.k);
}

constexpr size_t kMaxLds = 160 * 1024;
constexpr int kMaxTileChunks = 64;
// Tiles per workgroup of the weight-gradient kernels, at most: each lane
// adds its taps over the workgroup's tiles in fp32, one after another, and
// the rounding of such a run grows with its length; past this many tiles a
// channel gets more workgroups (and partial rows, summed in fp64).
constexpr int kMaxUnitsPerRow = 64;

hipError_t set_lds(const void* fn, size_t lds) { return prepare_lds(fn, lds); }

int resident(const void* fn, int nt, size_t lds) { return resident_wgs(fn, nt, lds); }

// Tiles per channel at the given tile size (default: the weight-gradient
// kernel's, the most of any tile kernel, which bounds the partial rows).
int tile_units_per_channel(const wtconv_shape& s, int th = kTileH, int tw = kTileW) {
    return s.B * ((s.H + th - 1) / th) * ((s.W + tw - 1) / tw);
}

int tile_chunks(const wtconv_shape& s, int slots, int units) {
    int want = slots / (s.C > 0 ? s.C : 1);
    if (want < 1) want = 1;
    if (want > kMaxTileChunks) want = kMaxTileChunks;
    if (want > units) want = units;
    int upw = (units + want - 1) / want;
    if (upw > kMaxUnitsPerRow) upw = kMaxUnitsPerRow;
    return (units + upw - 1) / upw;
}

// The most chunks tile_chunks returns for `units` tiles per channel, for any
// occupancy: what the workspace holds rows for.
int tile_chunk_bound(int units) {
    const int a = units < kMaxTileChunks ? units : kMaxTileChunks;
    const int b = (units + kMaxUnitsPerRow - 1) / kMaxUnitsPerRow;
    return a > b ? a : b;
}

template <typename T, int K>
const void* deep_apply_fn_k(bool flip) {
    return flip ? reinterpret_cast<const void*>(&k_deep_apply<T, K, true>)
                : reinterpret_cast<const void*>(&k_deep_apply<T, K, false>);
}

template <typename T>
const void* deep_apply_fn(bool flip, int k) {
    switch (k) {
        case 1: return deep_apply_fn_k<T, 1>(flip);
        case 3: return deep_apply_fn_k<T, 3>(flip);
        case 5: return deep_apply_fn_k<T, 5>(flip);
        default: return deep_apply_fn_k<T, 7>(flip);
    }
}

const void* deep_bww_fn(int k) {
    switch (k) {
        case 1: return reinterpret_cast<const void*>(&k_deep_bww<1>);
        case 3: return reinterpret_cast<const void*>(&k_deep_bww<3>);
        case 5: return reinterpret_cast<const void*>(&k_deep_bww<5>);
        default: return reinterpret_cast<const void*>(&k_deep_bww<7>);
    }
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
    // buffer offsets within a plane are 32-bit
    if (size_t(s.H) * size_t(s.W) * (s.dtype == WTCONV_F32 ? 4 : 2) >= (size_t(1) << 31))
        return false;
    return true;
}

// Workspace: [partial rows | deep contribution D | box sums P of x | of dy]
// (D and the box sums only with levels deeper than the tile's), then, when
// the deep levels run through device memory, [levels of x | of dy | conv
// outputs].
namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }
size_t p_bytes(const wtconv_shape& s) {
    const int LT = tile_lt(s);
    return size_t(s.B) * s.C * (s.H >> LT) * (s.W >> LT) * sizeof(float);
}
size_t rows_bytes(const wtconv_shape& s) {
    const int LT = tile_lt(s);
    const size_t KK = size_t(s.k) * s.k, npart = KK + 1 + 4 * size_t(s.L) * KK;
    const size_t chunks = size_t(tile_chunk_bound(tile_units_per_channel(s))) +
                          (s.L > LT ? size_t(s.B) : 0);
    return align_up(chunks * s.C * npart * sizeof(float));
}
float* d_of(const wtconv_shape& s, void* workspace) {
    return reinterpret_cast<float*>(static_cast<char*>(workspace) + rows_bytes(s));
}
float* p_of(const wtconv_shape& s, void* workspace, int which) {
    return reinterpret_cast<float*>(static_cast<char*>(workspace) + rows_bytes(s) +
                                    (1 + which) * align_up(p_bytes(s)));
}

// The deep levels stay in one workgroup's LDS when both deep kernels fit.
bool deep_in_lds(const wtconv_shape& s) {
    return deep_apply_lds(s) <= kMaxLds && deep_bww_lds(s) <= kMaxLds;
}
DeepGlobal deep_global(const wtconv_shape& s) {
    const int LT = tile_lt(s);
    return DeepGlobal{s.B * s.C, s.H >> LT, s.W >> LT, s.L - LT};
}
size_t g_bytes(const wtconv_shape& s) {
    const DeepGlobal G = deep_global(s);
    return align_up(G.level_off(G.LD + 1) * sizeof(float));
}
// 0: levels of P(x), 1: levels of P(dy), 2: conv outputs
float* g_of(const wtconv_shape& s, void* workspace, int which) {
    return reinterpret_cast<float*>(static_cast<char*>(workspace) + rows_bytes(s) +
                                    3 * align_up(p_bytes(s)) + which * g_bytes(s));
}
unsigned grid_for(size_t n) {
    const size_t g = (n + 255) / 256;
    return unsigned(g < 65536 ? g : 65536);
}

// Levels 1..LD of the box sums P into A (device-memory deep path).
hipError_t gdeep_analysis(const wtconv_shape& s, const float* P, float* A, hipStream_t stream) {
    const DeepGlobal G = deep_global(s);
    for (int m = 1; m <= G.LD; ++m) {
        const float* src = m == 1 ? P : A + G.level_off(m - 1);
        const size_t sps = m == 1 ? size_t(G.hp) * G.wp : size_t(4) * G.h(m - 1) * G.w(m - 1);
        const int sp = m == 1 ? G.wp : G.w(m - 1);
        const size_t n = size_t(G.planes) * G.h(m) * G.w(m);
        hipLaunchKernelGGL(k_gdeep_analysis, dim3(grid_for(n)), dim3(256), 0, stream, src, sps,
                           sp, A + G.level_off(m), G.planes, G.h(m), G.w(m));
    }
    return hipGetLastError();
}

template <typename T, int K>
const void* gdeep_conv_fn_k(bool flip) {
    return flip ? reinterpret_cast<const void*>(&k_gdeep_conv<T, K, true>)
                : reinterpret_cast<const void*>(&k_gdeep_conv<T, K, false>);
}
template <typename T, int K>
const void* gdeep_conv_lds_fn_k(bool flip) {
    return flip ? reinterpret_cast<const void*>(&k_gdeep_conv_lds<T, K, true>)
                : reinterpret_cast<const void*>(&k_gdeep_conv_lds<T, K, false>);
}
// The staged form where its LDS fits (lds > 0), else the direct one.
template <typename T>
const void* gdeep_conv_fn(bool flip, int k, size_t lds) {
    switch (k) {
        case 1: return lds ? gdeep_conv_lds_fn_k<T, 1>(flip) : gdeep_conv_fn_k<T, 1>(flip);
        case 3: return lds ? gdeep_conv_lds_fn_k<T, 3>(flip) : gdeep_conv_fn_k<T, 3>(flip);
        case 5: return lds ? gdeep_conv_lds_fn_k<T, 5>(flip) : gdeep_conv_fn_k<T, 5>(flip);
        default: return lds ? gdeep_conv_lds_fn_k<T, 7>(flip) : gdeep_conv_fn_k<T, 7>(flip);
    }
}
// Bytes of k_gdeep_conv_lds for an h x w level, or 0 past 64 KB.
size_t gdeep_conv_lds_bytes(int k, int h, int w) {
    const int p = k / 2, nseg = (w + kDeepRS - 1) / kDeepRS;
    const size_t bp = size_t((nseg * kDeepRS + 2 * p) | 1);
    const size_t b = sizeof(float) * (size_t(k) * k + (size_t(h) + 2 * p) * bp);
    return b <= 65536 ? b : 0;
}
// The staged form where its LDS fits (lds > 0), else the direct one.
const void* gdeep_corr_fn(int k, size_t lds) {
    switch (k) {
        case 1: return lds ? reinterpret_cast<const void*>(&k_gdeep_corr_lds<1>)
                           : reinterpret_cast<const void*>(&k_gdeep_corr<1>);
        case 3: return lds ? reinterpret_cast<const void*>(&k_gdeep_corr_lds<3>)
                           : reinterpret_cast<const void*>(&k_gdeep_corr<3>);
        case 5: return lds ? reinterpret_cast<const void*>(&k_gdeep_corr_lds<5>)
                           : reinterpret_cast<const void*>(&k_gdeep_corr<5>);
        default: return lds ? reinterpret_cast<const void*>(&k_gdeep_corr_lds<7>)
                            : reinterpret_cast<const void*>(&k_gdeep_corr<7>);
    }
}
// Bytes of k_gdeep_corr_lds for levels of at most h x w (level 1), or 0
// past 64 KB.
size_t gdeep_corr_lds_bytes(int k, int h, int w) {
    const int p = k / 2, nseg = (w + kDeepRS - 1) / kDeepRS;
    const size_t bpu = size_t((nseg * kDeepRS + 2 * p) | 1), bpv = size_t((nseg * kDeepRS) | 1);
    const size_t items = size_t(256 / k) * k;
    const size_t b = sizeof(float) * ((size_t(h) + 2 * p) * bpu + size_t(h) * bpv + items * k);
    return b <= 65536 ? b : 0;
}

// D from the levels A of the box sums: the convs of every level into Cb,
// each level folded into the LL below it, level 1 expanded over P's grid.
hipError_t gdeep_apply(const wtconv_shape& s, const float* A, const Params& p, bool flip,
                       float* Cb, float* deep, hipStream_t stream) {
    const DeepGlobal G = deep_global(s);
    const int LT = tile_lt(s);
    int C = s.C;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    for (int m = 1; m <= G.LD; ++m) {
        const float* u = A + G.level_off(m);
        float* o = Cb + G.level_off(m);
        int h = G.h(m), w = G.w(m), la = LT + m;
        const size_t lds = gdeep_conv_lds_bytes(s.k, h, w);
        const void* fn = s.dtype == WTCONV_F32 ? gdeep_conv_fn<float>(flip, s.k, lds)
                                               : gdeep_conv_fn<__half>(flip, s.k, lds);
        void* args[] = {&u, &o, &ww, &sw, &C, &h, &w, &la};
        hipError_t e = hipLaunchKernel(fn, dim3(unsigned(G.planes) * 4u), dim3(256), args,
                                       unsigned(lds), stream);
        if (e != hipSuccess) return e;
    }
    for (int m = G.LD; m >= 1; --m) {
        const size_t n = size_t(G.planes) * G.h(m - 1) * G.w(m - 1);
        float* dst = m > 1 ? Cb + G.level_off(m - 1) : deep;
        const size_t dps =
            m > 1 ? size_t(4) * G.h(m - 1) * G.w(m - 1) : size_t(G.hp) * G.wp;
        hipLaunchKernelGGL(k_gdeep_synth, dim3(grid_for(n)), dim3(256), 0, stream,
                           Cb + G.level_off(m), G.h(m), G.w(m), dst, dps, G.w(m - 1), G.planes,
                           m > 1);
    }
    return hipGetLastError();
}

// Deep partial rows (row0 + b) from the levels of both box sums.
hipError_t gdeep_rows(const wtconv_shape& s, const float* Ax, const float* Ady, float* part,
                      int row0, hipStream_t stream) {
    DeepGlobal G = deep_global(s);
    int C = s.C, LT = tile_lt(s), npart = s.k * s.k * (1 + 4 * s.L) + 1;
    void* args[] = {&Ax, &Ady, &G, &part, &C, &LT, &row0, &npart};
    const size_t lds = gdeep_corr_lds_bytes(s.k, G.h(1), G.w(1));
    const hipError_t e = hipLaunchKernel(gdeep_corr_fn(s.k, lds),
                                         dim3(unsigned(G.planes) * unsigned(G.LD) * 4u),
                                         dim3(256), args, unsigned(lds), stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_box_sums(const wtconv_shape& s, const void* src, float* P,
                           hipStream_t stream) {
    const int LT = tile_lt(s);
    const unsigned blocks = unsigned(size_t(s.B) * s.C * (s.H >> LT));
    if (s.dtype == WTCONV_F32)
        hipLaunchKernelGGL(k_box_sums<float>, dim3(blocks), dim3(128), 0, stream,
                           static_cast<const float*>(src), P, s.H, s.W, LT);
    else
        hipLaunchKernelGGL(k_box_sums<__half>, dim3(blocks), dim3(128), 0, stream,
                           static_cast<const __half*>(src), P, s.H, s.W, LT);
    return hipGetLastError();
}

// Deep levels' contribution D from the box sums P.
hipError_t launch_deep_apply(const wtconv_shape& s, const float* P, const Params& p, bool flip,
                             float* deep, hipStream_t stream) {
    const int LT = tile_lt(s);
    int B = s.B, C = s.C, H = s.H, W = s.W, L = s.L, LTv = LT;
    const void* fn = s.dtype == WTCONV_F32 ? deep_apply_fn<float>(flip, s.k)
                                           : deep_apply_fn<__half>(flip, s.k);
    const size_t lds = deep_apply_lds(s);
    hipError_t e;
    if ((e = set_lds(fn, lds)) != hipSuccess) return e;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    void* args[] = {&P, &ww, &sw, &deep, &B, &C, &H, &W, &L, &LTv};
    e = hipLaunchKernel(fn, dim3(unsigned(B) * unsigned(C)), dim3(kDeepNT), args, lds, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

// D from the box sums P on either deep path; on the device-memory path the
// levels of P are left in A.
hipError_t deep_contribution(const wtconv_shape& s, const float* P, const Params& p, bool flip,
                             float* deep, float* A, float* Cb, hipStream_t stream) {
    if (deep_in_lds(s)) return launch_deep_apply(s, P, p, flip, deep, stream);
    const hipError_t e = gdeep_analysis(s, P, A, stream);
    if (e != hipSuccess) return e;
    return gdeep_apply(s, A, p, flip, Cb, deep, stream);
}

// Deep partial rows from the box sums of x and dy on either path; Ady holds
// the levels of P(dy) already when `dy_levels`.
hipError_t deep_rows(const wtconv_shape& s, const float* Px, const float* Pdy, float* part,
                     int row0, void* workspace, bool dy_levels, hipStream_t stream) {
    hipError_t e;
    if (deep_in_lds(s)) {
        int B = s.B, C = s.C, H = s.H, W = s.W, L = s.L, LTv = tile_lt(s);
        int npart = s.k * s.k * (1 + 4 * s.L) + 1;
        const void* fn = deep_bww_fn(s.k);
        const size_t lds = deep_bww_lds(s);
        if ((e = set_lds(fn, lds)) != hipSuccess) return e;
        void* args[] = {&Px, &Pdy, &part, &B, &C, &H, &W, &L, &LTv, &row0, &npart};
        e = hipLaunchKernel(fn, dim3(unsigned(B) * unsigned(C)), dim3(kDeepNT), args, lds, stream);
        if (e != hipSuccess) return e;
        return hipGetLastError();
    }
    float* Ax = g_of(s, workspace, 0);
    float* Ady = g_of(s, workspace, 1);
    if ((e = gdeep_analysis(s, Px, Ax, stream)) != hipSuccess) return e;
    if (!dy_levels && (e = gdeep_analysis(s, Pdy, Ady, stream)) != hipSuccess) return e;
    return gdeep_rows(s, Ax, Ady, part, row0, stream);
}

// The tile kernels of the forward (flip = false) or input gradient, with the
// deep contribution (NULL: none).
hipError_t launch_tiles(const wtconv_shape& s, const TileVariant* v, const void* in,
                        const Params& p, void* out, bool flip, const float* deep,
                        hipStream_t stream) {
    int B = s.B, C = s.C, H = s.H, W = s.W;
    const void* fn = flip ? v->bwi : v->fwd;
    hipError_t e;
    if ((e = set_lds(fn, v->lds_apply)) != hipSuccess) return e;
    const long units = long(s.B) * ((s.H + v->ATH - 1) / v->ATH) * ((s.W + v->ATW - 1) / v->ATW);
    const long total = long(s.C) * units;
    long nwg = resident(fn, v->NT, v->lds_apply);
    if (nwg > total) nwg = total;
    const void* bb = flip ? p.w_base : p.b_base;  // read but unused when flipped
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

// Partial rows of the tiles and (with deeper levels) of the planes' deep
// levels, then the finalize.  Px, Pdy hold the box sums when L > LT.
hipError_t launch_weight_grads(const wtconv_shape& s, const TileVariant* v, const void* x,
                               const void* dy, const float* Px, const float* Pdy,
                               const Params& p, const Grads& g, void* workspace,
                               hipStream_t stream) {
    const int LT = tile_lt(s);
    hipError_t e;
    if ((e = set_lds(v->bww, v->lds_bww)) != hipSuccess) return e;
    const int units = tile_units_per_channel(s, v->TH, v->TW);
    const int nchunk = tile_chunks(s, resident(v->bww, v->NT, v->lds_bww), units);
    int upw = (units + nchunk - 1) / nchunk;
    int B = s.B, C = s.C, H = s.H, W = s.W;
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
        if ((e = deep_rows(s, Px, Pdy, part, nchunk, workspace, false, stream)) != hipSuccess)
            return e;
        rows += s.B;
    }
    return finalize_grads(s, part, rows, p, g, stream);
}
}  // namespace

size_t tile_workspace_bytes(const wtconv_shape& s) {
    if (!tile_supported(s) || s.B == 0 || s.C == 0) return 0;
    if (s.L <= tile_lt(s)) return rows_bytes(s);
    return rows_bytes(s) + 3 * align_up(p_bytes(s)) + (deep_in_lds(s) ? 0 : 3 * g_bytes(s));
}

hipError_t tile_apply(const wtconv_shape& s, const void* in, const Params& p, void* out,
                      bool flip, void* workspace, hipStream_t stream) {
    const TileVariant* v = find_tile(s);
    if (!v) return hipErrorInvalidValue;
    float* deep = nullptr;
    if (s.L > tile_lt(s)) {
        deep = d_of(s, workspace);
        float* P = p_of(s, workspace, 0);
        hipError_t e = launch_box_sums(s, in, P, stream);
        if (e == hipSuccess)
            e = deep_contribution(s, P, p, flip, deep, g_of(s, workspace, 0),
                                  g_of(s, workspace, 2), stream);
        if (e != hipSuccess) return e;
    }
    return launch_tiles(s, v, in, p, out, flip, deep, stream);
}

hipError_t tile_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                           const Params& p, const Grads& g, void* workspace,
                           hipStream_t stream) {
    const TileVariant* v = find_tile(s);
    if (!v) return hipErrorInvalidValue;
    float* Px = nullptr;
    float* Pdy = nullptr;
    if (s.L > tile_lt(s)) {
        Px = p_of(s, workspace, 0);
        Pdy = p_of(s, workspace, 1);
        hipError_t e = launch_box_sums(s, x, Px, stream);
        if (e == hipSuccess) e = launch_box_sums(s, dy, Pdy, stream);
        if (e != hipSuccess) return e;
    }
    return launch_weight_grads(s, v, x, dy, Px, Pdy, p, g, workspace, stream);
}

// Fused: with deeper levels, the box sums of dy and from them the deep input
// gradient D; then one pass over the tiles for dx, the tiles' weight
// partials and (deeper levels) the box sums of x; the deep levels' partials;
// the finalize.
hipError_t tile_bwd(const wtconv_shape& s, const void* x, const void* dy, const Params& p,
                    void* dx, const Grads& g, void* workspace, hipStream_t stream) {
    const TileVariant* v = find_tile(s);
    if (!v) return hipErrorInvalidValue;
    const int LT = tile_lt(s);
    hipError_t e;
    float* deep = nullptr;
    float* Px = nullptr;
    float* Pdy = nullptr;
    if (s.L > LT) {
        deep = d_of(s, workspace);
        Px = p_of(s, workspace, 0);
        Pdy = p_of(s, workspace, 1);
        if ((e = launch_box_sums(s, dy, Pdy, stream)) != hipSuccess) return e;
        if ((e = deep_contribution(s, Pdy, p, true, deep, g_of(s, workspace, 1),
                                   g_of(s, workspace, 2), stream)) != hipSuccess)
            return e;
    }
    if ((e = set_lds(v->bwd, v->lds_bwd)) != hipSuccess) return e;
    const int units = tile_units_per_channel(s, v->TH, v->BTW);
    const int nchunk = tile_chunks(s, resident(v->bwd, v->NT, v->lds_bwd), units);
    int upw = (units + nchunk - 1) / nchunk;
    int B = s.B, C = s.C, H = s.H, W = s.W;
    int npart = s.k * s.k * (1 + 4 * s.L) + 1;
    float* part = static_cast<float*>(workspace);
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    const float* dp = deep;
    {
        void* args[] = {&x,    &dy, &wb, &sb, &ww, &sw, &dp,  &dx,
                        &part, &Px, &B,  &C,  &H,  &W,  &upw, &npart};
        e = hipLaunchKernel(v->bwd, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                            v->lds_bwd, stream);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    int rows = nchunk;
    if (s.L > LT) {
        // the levels of P(dy) are in the workspace already on the device-memory
        // deep path (from the deep input gradient)
        if ((e = deep_rows(s, Px, Pdy, part, nchunk, workspace, true, stream)) != hipSuccess)
            return e;
        rows += s.B;
    }
    return finalize_grads(s, part, rows, p, g, stream);
}

}  // namespace wtc
