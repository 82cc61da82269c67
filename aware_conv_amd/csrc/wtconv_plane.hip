// Whole-plane fused WTConv kernels for gfx950.
//
// One workgroup owns one channel c and a group of P planes (b0..b0+P-1, same
// channel, so the same folded filters).  Everything between the HBM read of
// the input and the HBM write of the output stays in LDS and registers:
//
//   load      x planes -> LDS (fp32, zero border of width k/2 per level)
//   analysis  level l = 1..L: unnormalised signed 2x2 butterflies on the raw
//             LL of the level above, U^l_s = 2^l S^l_s ("recomputing the
//             Haar butterfly inside the depthwise conv kernel", gist.science/pt
//             "Metodologia"; the raw-LL recursion is the WTConv cascade)
//   convs     C^l_s = conv_{Wf[l,s]}(U^l_s) with folded filters
//             Wf[l,s] = gamma[l,c,s] * 4^-l * K[l,c,s], written over U^l_s
//   synthesis the per-level sign of each subband comes from bit l-1 of the
//             output coordinates (the closed-form, bit-indexed synthesis of
//             the same section): coarse levels are folded into the LL of the
//             next finer level, level 1 is expanded per output pixel
//   output    y = conv_{beta*Kb}(x) + beta*bias + level-1 synthesis -> HBM
//
// The folded filters are the "scale folding" of the same section: gamma and
// beta multiply the filters, beta the bias, and the Haar factors 1/2 of
// analysis and synthesis give the extra 4^-l (derivation in the design notes).
// The input gradient runs the same kernel with every filter rotated by 180
// degrees and no bias: the layer minus its bias is linear and this is its
// transpose.
//
// The weight-gradient kernel recomputes the same analysis of x and of dy and
// accumulates G_b[u,v] = sum dy * x(shifted), sum dy, and
// G[l,s][u,v] = sum V^l_s(dy) * U^l_s(x)(shifted) in registers across the
// workgroup's planes, reduces them with wave64 shuffles and LDS, and writes one
// fp32 partial row per workgroup; a finalize kernel sums the partial rows in a
// fixed order and applies the chain rule through the fold.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "wtconv_internal.h"

namespace wtc {
namespace {

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(__half v) { return __half2float(v); }
template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ float from_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ __half from_f<__half>(float v) {
    return __float2half_rn(v);
}

// Register tile of a conv phase: each work item computes Q rows x R columns.
struct Tile {
    int R, Q;
};

// Pick (R, Q) for an output grid of rows x cols repeated `count` times:
// fewest wave-issue slots for the FMA sweep plus the LDS reads, with at most
// `maxacc` live accumulators per thread.
constexpr Tile pick_tile(int rows, int cols, int count, int K, int NT,
                         int maxacc) {
    Tile best{1, 1};
    double bestc = 1e300;
    const int Rs[8] = {8, 7, 6, 5, 4, 3, 2, 1};
    const int Qs[3] = {4, 2, 1};
    for (int a = 0; a < 8; ++a) {
        int R = Rs[a];
        if (cols % R) continue;
        for (int b = 0; b < 3; ++b) {
            int Q = Qs[b];
            if (rows % Q) continue;
            if (Q * R > 16) continue;
            int items = count * (rows / Q) * (cols / R);
            int rounds = cdiv(items, NT);
            if (rounds * Q * R > maxacc) continue;
            double ic = double(Q * R * K * K) +
                        0.5 * double((Q + K - 1) * (R + K - 1) + K * K);
            double c = double(cdiv(items, 64)) * ic +
                       0.25 * double(rounds) * ic * double(NT / 64);
            if (c < bestc) {
                bestc = c;
                best = Tile{R, Q};
            }
        }
    }
    return best;
}

// LDS geometry of a group of P planes.  Level 0 holds the input planes;
// level l >= 1 holds the four subbands of each plane.  Every 2-D array has a
// zero border of p = k/2 rows top and bottom and at least p columns left and
// right; the interior starts at column OX so that rows stay 16-byte aligned.
template <int K_, int L_, int H_, int W_, int P_, int NT_>
struct Geo {
    static constexpr int K = K_, L = L_, H = H_, W = W_, P = P_, NT = NT_;
    static constexpr int p = K / 2, KK = K * K;
    static constexpr int OX = 4;
    __host__ __device__ static constexpr int hl(int l) { return H >> l; }
    __host__ __device__ static constexpr int wl(int l) { return W >> l; }
    __host__ __device__ static constexpr int pitch(int l) {
        int q = (OX + wl(l) + 4 + 3) & ~3;
        if (q % 32 == 0) q += 4;
        return q;
    }
    __host__ __device__ static constexpr int rows(int l) { return hl(l) + 2 * p; }
    __host__ __device__ static constexpr int arr(int l) { return rows(l) * pitch(l); }
    __host__ __device__ static constexpr int nsub(int l) { return l == 0 ? 1 : 4; }
    __host__ __device__ static constexpr int region(int l) { return P * nsub(l) * arr(l); }
    __host__ __device__ static constexpr int off(int l) {
        int o = 0;
        for (int m = 0; m < l; ++m) o += region(m);
        return o;
    }
    static constexpr int side = off(L + 1);           // floats of one side
    static constexpr int NWF = KK * (1 + 4 * L) + 1;  // folded filters + bias
    static constexpr int NPART = KK + 1 + 4 * L * KK; // weight-gradient row
    // Interior element (i, j) of array (level l, plane pl, subband s); i and
    // j may reach into the border (down to -p).
    __host__ __device__ static constexpr int idx(int l, int pl, int s, int i,
                                                 int j) {
        return off(l) + (pl * nsub(l) + s) * arr(l) + (i + p) * pitch(l) + OX + j;
    }
    static_assert((H % (1 << L)) == 0 && (W % (1 << L)) == 0, "H, W % 2^L");
    static_assert(NT % 64 == 0, "whole waves");
};

// Widest vector (in elements, at most 16 bytes) that divides n.
template <typename T>
constexpr int vec_elems(int n) {
    constexpr int maxv = 16 / int(sizeof(T));
    int v = maxv;
    while (v > 1 && (n % v)) v /= 2;
    return v;
}

template <typename T, int V>
__device__ __forceinline__ void load_vec(const T* __restrict__ src, float (&v)[V]) {
    if constexpr (std::is_same<T, float>::value && V == 4) {
        float4 q = *reinterpret_cast<const float4*>(src);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else if constexpr (std::is_same<T, __half>::value && V == 8) {
        union { uint4 u; __half2 h[4]; } pk;
        pk.u = *reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float2 f = __half22float2(pk.h[e]);
            v[2 * e] = f.x;
            v[2 * e + 1] = f.y;
        }
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = to_f(src[e]);
    }
}

template <typename T, int V>
__device__ __forceinline__ void store_vec(T* __restrict__ dst, const float* v) {
    if constexpr (std::is_same<T, float>::value && V == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (std::is_same<T, float>::value && V == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
    } else if constexpr (std::is_same<T, __half>::value && V == 8) {
        union { uint4 u; __half2 h[4]; } pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk.h[e] = __floats2half2_rn(v[2 * e], v[2 * e + 1]);
        *reinterpret_cast<uint4*>(dst) = pk.u;
    } else if constexpr (std::is_same<T, __half>::value && V == 4) {
        union { uint2 u; __half2 h[2]; } pk;
        pk.h[0] = __floats2half2_rn(v[0], v[1]);
        pk.h[1] = __floats2half2_rn(v[2], v[3]);
        *reinterpret_cast<uint2*>(dst) = pk.u;
    } else if constexpr (std::is_same<T, __half>::value && V == 2) {
        *reinterpret_cast<__half2*>(dst) = __floats2half2_rn(v[0], v[1]);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) dst[e] = from_f<T>(v[e]);
    }
}

// ---------------------------------------------------------------------------
// Phases
// ---------------------------------------------------------------------------

// HBM -> LDS interior of level 0 for planes b0..b0+P-1 (zeros past B).
template <class G, typename T>
__device__ __forceinline__ void load_planes(float* lds, const T* __restrict__ src,
                                            int b0, int B, int C, int c, int tid) {
    constexpr int V = vec_elems<T>(G::W);
    constexpr int NV = G::W / V;
    constexpr int ITEMS = G::P * G::H * NV;
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int cv = item % NV;
            const int r = (item / NV) % G::H;
            const int pl = item / (NV * G::H);
            const int b = b0 + pl;
            float v[V];
            if (b < B) {
                const T* s = src + ((size_t(b) * C + c) * G::H + r) * G::W + cv * V;
                load_vec<T, V>(s, v);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) v[e] = 0.f;
            }
            float* d = lds + G::idx(0, pl, 0, r, cv * V);
            if constexpr (V % 4 == 0) {
#pragma unroll
                for (int e = 0; e < V; e += 4)
                    *reinterpret_cast<float4*>(d + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) d[e] = v[e];
            }
        }
    }
}

// Level-l analysis from the raw LL of level l-1 (the input plane at l = 1):
// (a, b; c, d) -> LL = a+b+c+d, LH = a-b+c-d, HL = a+b-c-d, HH = a-b-c+d.
template <class G, int l>
__device__ __forceinline__ void analysis_level(float* lds, int tid) {
    constexpr int h = G::hl(l), w = G::wl(l), ITEMS = G::P * h * w;
    constexpr int sp = G::pitch(l - 1), A = G::arr(l);
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int j = item % w;
            const int i = (item / w) % h;
            const int pl = item / (w * h);
            const float* s = lds + G::idx(l - 1, pl, 0, 2 * i, 2 * j);
            const float a = s[0], b = s[1], c = s[sp], d = s[sp + 1];
            const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
            float* o = lds + G::idx(l, pl, 0, i, j);
            o[0] = s0 + s1;
            o[A] = d0 + d1;
            o[2 * A] = s0 - s1;
            o[3 * A] = d0 - d1;
        }
    }
}

// acc[q][j] = sum_{u,v} w[u*K+v] * src[(q+u)*PITCH + j+v]: a Q x R tile of a
// 'same' cross-correlation whose window's top-left element is src.
template <int K, int Q, int R, int PITCH>
__device__ __forceinline__ void conv_tile(const float* src, const float* wk,
                                          float (&acc)[Q][R]) {
    float w[K * K];
#pragma unroll
    for (int t = 0; t < K * K; ++t) w[t] = wk[t];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[q][j] = 0.f;
#pragma unroll
    for (int ir = 0; ir < Q + K - 1; ++ir) {
        float in[R + K - 1];
#pragma unroll
        for (int m = 0; m < R + K - 1; ++m) in[m] = src[ir * PITCH + m];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int j = 0; j < R; ++j)
                        acc[q][j] = fmaf(w[u * K + v], in[j + v], acc[q][j]);
            }
        }
    }
}

// C^l_s = conv(U^l_s) for all planes and subbands, written over U^l_s.
template <class G, int l>
__device__ __forceinline__ void conv_level(float* lds, const float* wf, int tid) {
    constexpr int h = G::hl(l), w = G::wl(l);
    constexpr Tile T = pick_tile(h, w, G::P * 4, G::K, G::NT, 16);
    constexpr int R = T.R, Q = T.Q, NS = w / R, NQ = h / Q;
    constexpr int ITEMS = G::P * 4 * NQ * NS, MAXI = cdiv(ITEMS, G::NT);
    constexpr int PITCH = G::pitch(l);
    float res[MAXI][Q][R];
#pragma unroll
    for (int it = 0; it < MAXI; ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int s = item & 3;
            int r = item >> 2;
            const int strip = r % NS;
            r /= NS;
            const int qi = r % NQ;
            const int pl = r / NQ;
            const float* src = lds + G::idx(l, pl, s, qi * Q - G::p, strip * R - G::p);
            conv_tile<G::K, Q, R, PITCH>(src, wf + G::KK * (1 + (l - 1) * 4 + s), res[it]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < MAXI; ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int s = item & 3;
            int r = item >> 2;
            const int strip = r % NS;
            r /= NS;
            const int qi = r % NQ;
            const int pl = r / NQ;
            float* dst = lds + G::idx(l, pl, s, qi * Q, strip * R);
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int j = 0; j < R; ++j) dst[q * PITCH + j] = res[it][q][j];
        }
    }
}

// Fold level l's convolved subbands into the LL of level l-1: each coarse
// coefficient lands on the 2x2 block below it with the sign of its subband at
// the block position (row bit for HL, column bit for LH, both for HH).
template <class G, int l>
__device__ __forceinline__ void cascade_level(float* lds, int tid) {
    constexpr int h = G::hl(l - 1), w = G::wl(l - 1), ITEMS = G::P * h * w;
    constexpr int A = G::arr(l);
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int j = item % w;
            const int i = (item / w) % h;
            const int pl = item / (w * h);
            const float* cs = lds + G::idx(l, pl, 0, i >> 1, j >> 1);
            const float sy = (i & 1) ? -1.f : 1.f, sx = (j & 1) ? -1.f : 1.f;
            const float e = fmaf(sy, cs[2 * A], cs[0]);
            const float f = fmaf(sy, cs[3 * A], cs[A]);
            lds[G::idx(l - 1, pl, 0, i, j)] += fmaf(sx, f, e);
        }
    }
}

// Base conv plus bias plus the level-1 synthesis, then the HBM store.
template <class G, typename T>
__device__ __forceinline__ void final_out(const float* lds, const float* wf,
                                          T* __restrict__ out, int b0, int B,
                                          int C, int c, int tid) {
    constexpr Tile T0 = pick_tile(G::H, G::W, G::P, G::K, G::NT, 32);
    constexpr int R = T0.R, Q = T0.Q, NS = G::W / R, NQ = G::H / Q;
    constexpr int ITEMS = G::P * NQ * NS;
    constexpr int A1 = G::arr(1);
    constexpr int VS = vec_elems<T>(R) < vec_elems<T>(G::W) ? vec_elems<T>(R) : vec_elems<T>(G::W);
    const float bias = wf[G::NWF - 1];
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int strip = item % NS;
            const int qi = (item / NS) % NQ;
            const int pl = item / (NS * NQ);
            float acc[Q][R];
            conv_tile<G::K, Q, R, G::pitch(0)>(
                lds + G::idx(0, pl, 0, qi * Q - G::p, strip * R - G::p), wf, acc);
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int yy = qi * Q + q;
                const float sy = (yy & 1) ? -1.f : 1.f;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int xx = strip * R + j;
                    const float sx = (xx & 1) ? -1.f : 1.f;
                    const float* cs = lds + G::idx(1, pl, 0, yy >> 1, xx >> 1);
                    const float e = fmaf(sy, cs[2 * A1], cs[0]);
                    const float f = fmaf(sy, cs[3 * A1], cs[A1]);
                    acc[q][j] += bias + fmaf(sx, f, e);
                }
            }
            const int b = b0 + pl;
            if (b < B) {
                T* dst = out + ((size_t(b) * C + c) * G::H + qi * Q) * G::W + strip * R;
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int j = 0; j < R; j += VS)
                        store_vec<T, VS>(dst + q * G::W + j, &acc[q][j]);
            }
        }
    }
}

// Folded filters in LDS: [0, KK) base, then (l, s) blocks, then the bias.
template <class G, typename T, bool FLIP>
__device__ __forceinline__ void fold_weights(float* wf, const T* __restrict__ wb,
                                             const T* __restrict__ bb,
                                             const T* __restrict__ sb,
                                             const T* __restrict__ ww,
                                             const T* __restrict__ sw, int C,
                                             int c, int tid) {
    constexpr int KK = G::KK;
    for (int i = tid; i < G::NWF; i += G::NT) {
        float v;
        if (i < KK) {
            const int t = FLIP ? KK - 1 - i : i;
            v = to_f(sb[c]) * to_f(wb[size_t(c) * KK + t]);
        } else if (i < G::NWF - 1) {
            const int jj = i - KK, ls = jj / KK, t = jj % KK;
            const int l = ls >> 2, s = ls & 3;
            const int tt = FLIP ? KK - 1 - t : t;
            const size_t gi = (size_t(l) * C + c) * 4 + s;
            v = to_f(sw[gi]) * ldexpf(1.f, -2 * (l + 1)) * to_f(ww[gi * KK + tt]);
        } else {
            v = FLIP ? 0.f : to_f(sb[c]) * to_f(bb[c]);
        }
        wf[i] = v;
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Forward (FLIP = false) or input gradient (FLIP = true) of planes of
// channel blockIdx.x % C; the workgroup covers `gpw` groups of P planes.
template <int K, int L, int H, int W, int P, int NT, typename T, bool FLIP>
__global__ __launch_bounds__(NT) void k_plane_apply(
    const T* __restrict__ in, const T* __restrict__ wb, const T* __restrict__ bb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    T* __restrict__ out, int B, int C, int gpw) {
    using G = Geo<K, L, H, W, P, NT>;
    extern __shared__ float lds[];
    float* wf = lds + G::side;
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    for (int i = tid; i < G::side; i += NT) lds[i] = 0.f;
    fold_weights<G, T, FLIP>(wf, wb, bb, sb, ww, sw, C, c, tid);
    __syncthreads();
    const int ngroups = cdiv(B, P);
    const int g0 = chunk * gpw;
    const int g1 = min(g0 + gpw, ngroups);
    for (int g = g0; g < g1; ++g) {
        const int b0 = g * P;
        load_planes<G, T>(lds, in, b0, B, C, c, tid);
        __syncthreads();
        static_for<1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value>(lds, tid);
            __syncthreads();
        });
        static_for<1, L + 1>([&](auto lc) { conv_level<G, decltype(lc)::value>(lds, wf, tid); });
        __syncthreads();
        static_for<0, L - 1>([&](auto lc) {
            cascade_level<G, L - decltype(lc)::value>(lds, tid);
            __syncthreads();
        });
        final_out<G, T>(lds, wf, out, b0, B, C, c, tid);
        __syncthreads();
    }
}

// Correlation accumulation of one Q x R tile: acc[u*K+v] += sum_{q,j}
// d[q][j] * src[(q+u)*PITCH + j+v].
template <int K, int Q, int R, int PITCH>
__device__ __forceinline__ void corr_tile(const float (&d)[Q][R], const float* src,
                                          float (&acc)[K * K]) {
#pragma unroll
    for (int ir = 0; ir < Q + K - 1; ++ir) {
        float in[R + K - 1];
#pragma unroll
        for (int m = 0; m < R + K - 1; ++m) in[m] = src[ir * PITCH + m];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int j = 0; j < R; ++j)
                        acc[u * K + v] = fmaf(d[q][j], in[j + v], acc[u * K + v]);
            }
        }
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Weight-gradient partial sums of channel blockIdx.x % C over the groups of
// chunk blockIdx.x / C: one row of G::NPART floats per workgroup,
// [G_b (KK), sum dy, G[l][s] (4 L KK)].
template <int K, int L, int H, int W, int P, int NT, typename T>
__global__ __launch_bounds__(NT) void k_plane_bww(
    const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ part,
    int B, int C, int gpw) {
    using G = Geo<K, L, H, W, P, NT>;
    constexpr int KK = G::KK;
    extern __shared__ float lds[];
    float* lx = lds;
    float* ld = lds + G::side;
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    for (int i = tid; i < 2 * G::side; i += NT) lds[i] = 0.f;
    __syncthreads();
    float accB[KK], accL[L][KK], sdy = 0.f;
#pragma unroll
    for (int t = 0; t < KK; ++t) accB[t] = 0.f;
#pragma unroll
    for (int l = 0; l < L; ++l)
#pragma unroll
        for (int t = 0; t < KK; ++t) accL[l][t] = 0.f;

    const int ngroups = cdiv(B, P);
    const int g0 = chunk * gpw;
    const int g1 = min(g0 + gpw, ngroups);
    for (int g = g0; g < g1; ++g) {
        const int b0 = g * P;
        load_planes<G, T>(lx, x, b0, B, C, c, tid);
        load_planes<G, T>(ld, dy, b0, B, C, c, tid);
        __syncthreads();
        static_for<1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value>(lx, tid);
            analysis_level<G, decltype(lc)::value>(ld, tid);
            __syncthreads();
        });
        // base path: G_b and sum dy
        {
            constexpr Tile T0 = pick_tile(H, W, P, K, NT, 32);
            constexpr int R = T0.R, Q = T0.Q, NS = W / R, NQ = H / Q;
            constexpr int ITEMS = P * NQ * NS;
#pragma unroll
            for (int it = 0; it < cdiv(ITEMS, NT); ++it) {
                const int item = tid + it * NT;
                if (ITEMS % NT == 0 || item < ITEMS) {
                    const int strip = item % NS;
                    const int qi = (item / NS) % NQ;
                    const int pl = item / (NS * NQ);
                    float d[Q][R];
                    const float* ds = ld + G::idx(0, pl, 0, qi * Q, strip * R);
#pragma unroll
                    for (int q = 0; q < Q; ++q)
#pragma unroll
                        for (int j = 0; j < R; ++j) {
                            d[q][j] = ds[q * G::pitch(0) + j];
                            sdy += d[q][j];
                        }
                    corr_tile<K, Q, R, G::pitch(0)>(
                        d, lx + G::idx(0, pl, 0, qi * Q - G::p, strip * R - G::p), accB);
                }
            }
        }
        // wavelet levels: the subband of every item of this thread is tid & 3
        static_for<1, L + 1>([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            constexpr int h = G::hl(l), w = G::wl(l);
            constexpr Tile TT = pick_tile(h, w, P * 4, K, NT, 32);
            constexpr int R = TT.R, Q = TT.Q, NS = w / R, NQ = h / Q;
            constexpr int ITEMS = P * 4 * NQ * NS;
#pragma unroll
            for (int it = 0; it < cdiv(ITEMS, NT); ++it) {
                const int item = tid + it * NT;
                if (ITEMS % NT == 0 || item < ITEMS) {
                    const int s = item & 3;
                    int r = item >> 2;
                    const int strip = r % NS;
                    r /= NS;
                    const int qi = r % NQ;
                    const int pl = r / NQ;
                    float d[Q][R];
                    const float* vs = ld + G::idx(l, pl, s, qi * Q, strip * R);
#pragma unroll
                    for (int q = 0; q < Q; ++q)
#pragma unroll
                        for (int j = 0; j < R; ++j) d[q][j] = vs[q * G::pitch(l) + j];
                    corr_tile<K, Q, R, G::pitch(l)>(
                        d, lx + G::idx(l, pl, s, qi * Q - G::p, strip * R - G::p), accL[l - 1]);
                }
            }
        });
        __syncthreads();
    }

    // workgroup reduction in a fixed order
    constexpr int NWAVES = NT / 64;
    constexpr int NPART = G::NPART;
    const int lane = tid & 63, wv = tid >> 6;
    float* red = lds;
#pragma unroll
    for (int t = 0; t < KK; ++t) {
        const float v = wave_sum(accB[t]);
        if (lane == 0) red[wv * NPART + t] = v;
    }
    {
        const float v = wave_sum(sdy);
        if (lane == 0) red[wv * NPART + KK] = v;
    }
#pragma unroll
    for (int l = 0; l < L; ++l)
#pragma unroll
        for (int t = 0; t < KK; ++t) {
            float v = accL[l][t];
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (lane < 4) red[wv * NPART + KK + 1 + (l * 4 + lane) * KK + t] = v;
        }
    __syncthreads();
    for (int i = tid; i < NPART; i += NT) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) s += red[w * NPART + i];
        part[(size_t(chunk) * C + c) * NPART + i] = s;
    }
}

// Sum the partial rows of every chunk in order and apply the chain rule
// through the fold: dKb = beta G_b, dbias = beta sum dy,
// dbeta = <Kb, G_b> + bias sum dy, dK[l,s] = gamma 4^-l G[l,s],
// dgamma[l,s] = 4^-l <K[l,s], G[l,s]>.  nchunk = 0 gives zero gradients.
template <typename T>
__global__ void k_bww_final(const float* __restrict__ part, int nchunk, int C,
                            int K, int L, const T* __restrict__ wb,
                            const T* __restrict__ bb, const T* __restrict__ sb,
                            const T* __restrict__ ww, const T* __restrict__ sw,
                            T* __restrict__ dwb, T* __restrict__ dbb,
                            T* __restrict__ dsb, T* __restrict__ dww,
                            T* __restrict__ dsw) {
    extern __shared__ float g[];
    const int KK = K * K, NPART = KK + 1 + 4 * L * KK;
    const int c = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    for (int i = tid; i < NPART; i += nt) {
        float s = 0.f;
        for (int ch = 0; ch < nchunk; ++ch) s += part[(size_t(ch) * C + c) * NPART + i];
        g[i] = s;
    }
    __syncthreads();
    const float beta = to_f(sb[c]);
    for (int i = tid; i < KK; i += nt) dwb[size_t(c) * KK + i] = from_f<T>(beta * g[i]);
    if (tid == 0) {
        dbb[c] = from_f<T>(beta * g[KK]);
        float dot = 0.f;
        for (int t = 0; t < KK; ++t) dot = fmaf(to_f(wb[size_t(c) * KK + t]), g[t], dot);
        dsb[c] = from_f<T>(fmaf(to_f(bb[c]), g[KK], dot));
    }
    for (int i = tid; i < 4 * L * KK; i += nt) {
        const int ls = i / KK, t = i % KK, l = ls >> 2, s = ls & 3;
        const size_t gi = (size_t(l) * C + c) * 4 + s;
        dww[gi * KK + t] = from_f<T>(to_f(sw[gi]) * ldexpf(1.f, -2 * (l + 1)) * g[KK + 1 + i]);
    }
    for (int i = tid; i < 4 * L; i += nt) {
        const int l = i >> 2, s = i & 3;
        const size_t gi = (size_t(l) * C + c) * 4 + s;
        float dot = 0.f;
        for (int t = 0; t < KK; ++t) dot = fmaf(to_f(ww[gi * KK + t]), g[KK + 1 + i * KK + t], dot);
        dsw[gi] = from_f<T>(ldexpf(1.f, -2 * (l + 1)) * dot);
    }
}

// ---------------------------------------------------------------------------
// Variant table
// ---------------------------------------------------------------------------

struct Variant {
    int K, L, H, W, dtype, P, NT;
    const void* fwd;
    const void* bwi;
    const void* bww;
    size_t lds_apply, lds_bww;
};

template <int K, int L, int H, int W, int P, int NT, typename T>
Variant make_variant(int dtype) {
    using G = Geo<K, L, H, W, P, NT>;
    size_t la = sizeof(float) * (G::side + G::NWF);
    size_t lb = sizeof(float) * (2 * G::side);
    size_t lr = sizeof(float) * (NT / 64) * G::NPART;
    if (lb < lr) lb = lr;
    return Variant{K, L, H, W, dtype, P, NT,
                   reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, false>),
                   reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, true>),
                   reinterpret_cast<const void*>(&k_plane_bww<K, L, H, W, P, NT, T>),
                   la, lb};
}

// (K, L, H, W, planes per workgroup, threads).  The ConvNeXt-T stage shapes
// first, then small shapes for edge cases.
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
    X(5, 6, 64, 64, 1, 256)

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

// Groups per workgroup for the weight-gradient pass: enough workgroups to fill
// the chip about twice, each covering a contiguous run of groups.
int bww_gpw(const wtconv_shape& s, int P) {
    const int ngroups = cdiv(s.B, P);
    const long total = long(ngroups) * s.C;
    const long target = 1024;
    int gpw = int((total + target - 1) / target);
    if (gpw < 1) gpw = 1;
    if (gpw > ngroups) gpw = ngroups > 0 ? ngroups : 1;
    return gpw;
}

}  // namespace

bool plane_supported(const wtconv_shape& s) { return find_variant(s) != nullptr; }

size_t plane_workspace_bytes(const wtconv_shape& s) {
    const Variant* v = find_variant(s);
    if (!v || s.B == 0 || s.C == 0) return 0;
    const int gpw = bww_gpw(s, v->P);
    const int nchunk = cdiv(cdiv(s.B, v->P), gpw);
    const int KK = s.k * s.k;
    const size_t npart = size_t(KK) + 1 + size_t(4) * s.L * KK;
    return size_t(nchunk) * s.C * npart * sizeof(float);
}

hipError_t plane_apply(const wtconv_shape& s, const void* in, const Params& p,
                       void* out, bool flip, hipStream_t stream) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    const void* fn = flip ? v->bwi : v->fwd;
    hipError_t e = prepare(fn, v->lds_apply);
    if (e != hipSuccess) return e;
    const int ngroups = cdiv(s.B, v->P);
    int gpw = 1, B = s.B, C = s.C;
    const int nchunk = ngroups;
    const void* bb = flip ? p.w_base : p.b_base;  // unread when flipped
    const void* wb = p.w_base;
    const void* sb = p.s_base;
    const void* ww = p.w_wav;
    const void* sw = p.s_wav;
    void* args[] = {&in, &wb, &bb, &sb, &ww, &sw, &out, &B, &C, &gpw};
    e = hipLaunchKernel(fn, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                        v->lds_apply, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t plane_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                            const Params& p, const Grads& g, void* workspace,
                            hipStream_t stream) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    hipError_t e = prepare(v->bww, v->lds_bww);
    if (e != hipSuccess) return e;
    int gpw = bww_gpw(s, v->P), B = s.B, C = s.C;
    const int nchunk = cdiv(cdiv(s.B, v->P), gpw);
    float* part = static_cast<float*>(workspace);
    void* args[] = {&x, &dy, &part, &B, &C, &gpw};
    e = hipLaunchKernel(v->bww, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                        v->lds_bww, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int KK = s.k * s.k;
    const size_t lds = sizeof(float) * (size_t(KK) + 1 + size_t(4) * s.L * KK);
    if (s.dtype == WTCONV_F32) {
        hipLaunchKernelGGL(k_bww_final<float>, dim3(s.C), dim3(256), lds, stream,
                           static_cast<const float*>(workspace), nchunk, s.C, s.k, s.L,
                           (const float*)p.w_base, (const float*)p.b_base,
                           (const float*)p.s_base, (const float*)p.w_wav,
                           (const float*)p.s_wav, (float*)g.dw_base, (float*)g.db_base,
                           (float*)g.ds_base, (float*)g.dw_wav, (float*)g.ds_wav);
    } else {
        hipLaunchKernelGGL(k_bww_final<__half>, dim3(s.C), dim3(256), lds, stream,
                           static_cast<const float*>(workspace), nchunk, s.C, s.k, s.L,
                           (const __half*)p.w_base, (const __half*)p.b_base,
                           (const __half*)p.s_base, (const __half*)p.w_wav,
                           (const __half*)p.s_wav, (__half*)g.dw_base, (__half*)g.db_base,
                           (__half*)g.ds_base, (__half*)g.dw_wav, (__half*)g.ds_wav);
    }
    return hipGetLastError();
}

hipError_t zero_grads(const wtconv_shape& s, const Params& p, const Grads& g,
                      hipStream_t stream) {
    const int KK = s.k * s.k;
    const size_t lds = sizeof(float) * (size_t(KK) + 1 + size_t(4) * s.L * KK);
    if (s.dtype == WTCONV_F32) {
        hipLaunchKernelGGL(k_bww_final<float>, dim3(s.C), dim3(256), lds, stream,
                           nullptr, 0, s.C, s.k, s.L, (const float*)p.w_base,
                           (const float*)p.b_base, (const float*)p.s_base,
                           (const float*)p.w_wav, (const float*)p.s_wav,
                           (float*)g.dw_base, (float*)g.db_base, (float*)g.ds_base,
                           (float*)g.dw_wav, (float*)g.ds_wav);
    } else {
        hipLaunchKernelGGL(k_bww_final<__half>, dim3(s.C), dim3(256), lds, stream,
                           nullptr, 0, s.C, s.k, s.L, (const __half*)p.w_base,
                           (const __half*)p.b_base, (const __half*)p.s_base,
                           (const __half*)p.w_wav, (const __half*)p.s_wav,
                           (__half*)g.dw_base, (__half*)g.db_base, (__half*)g.ds_base,
                           (__half*)g.dw_wav, (__half*)g.ds_wav);
    }
    return hipGetLastError();
}

}  // namespace wtc
