// Whole-plane fused WTConv kernels for gfx950.
//
// One workgroup owns one channel c and walks over groups of P planes
// (b0..b0+P-1, all of channel c, so all sharing the same folded filters).
// Everything between the HBM read of the input and the HBM write of the
// output stays in LDS and registers:
//
//   load      x planes -> LDS (fp32) and, from the same registers, the level-1
//             Haar butterflies: unnormalised signed 2x2 sums U^1_s = 2 S^1_s
//             ("recomputing the Haar butterfly inside the depthwise conv
//             kernel", gist.science/pt "Metodologia")
//   analysis  levels l = 2..L from the raw LL of the level above (the WTConv
//             cascade analyses the raw LL), U^l_s = 2^l S^l_s
//   convs     every lane owns one Q x R output tile of one array: the base
//             conv of a plane, or one subband of one level.  The same code
//             path serves every level, so a wavefront never splits across
//             levels; filters are folded (gamma * 4^-l * K, beta * Kb) and
//             sit in VGPRs for the whole kernel
//   synthesis results overwrite their inputs in LDS; each coarse level is
//             folded into the LL of the next finer level with the sign its
//             subband has at the 2x2 position (bit l-1 of the output
//             coordinates: the closed-form, bit-indexed synthesis of the same
//             section), then level 1 is expanded per output pixel, added to
//             the base conv and the bias, and stored
//
// The input gradient runs the same kernel with every filter rotated by 180
// degrees and no bias: the layer minus its bias is linear and that is its
// transpose.
//
// The weight-gradient kernel recomputes the same analysis of x and of dy.
// Each lane owns the same tile position on every plane of its workgroup and
// accumulates the k*k correlation taps of that tile (base: dy against x;
// level l subband s: V^l_s(dy) against U^l_s(x)) in registers across all the
// planes; the workgroup then sums the lanes of each (array, subband) in a
// fixed order and writes one fp32 partial row.  A finalize kernel sums the
// rows of the batch chunks in order and applies the chain rule through the
// fold, so results are bitwise reproducible.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ---------------------------------------------------------------------------
// Work decomposition
// ---------------------------------------------------------------------------

struct Tile {
    int R, Q;  // columns and rows of one lane's output tile
    int jobs;  // tiles per group of planes, over all levels
};

__host__ __device__ constexpr int njobs(int K, int L, int H, int W, int P, int R, int Q) {
    int n = 0;
    for (int l = 0; l <= L; ++l)
        n += P * (l ? 4 : 1) * cdiv(W >> l, R) * cdiv(H >> l, Q);
    return n;
}

// The tile that gives every lane the least work (Q*R outputs, k*k FMAs each)
// with one tile per lane; ties go to the tile with fewer LDS reads per FMA.
constexpr Tile plan_tile(int K, int L, int H, int W, int P, int NT, int maxqr) {
    Tile best{0, 0, 0};
    double bc = 1e300;
    for (int R = 1; R <= 8; ++R)
        for (int Q = 1; Q <= 8; ++Q) {
            if (Q * R > maxqr) continue;
            const int n = njobs(K, L, H, W, P, R, Q);
            if (n > NT) continue;
            const double reads = double((Q + K - 1) * (R + K - 1)) / double(Q * R * K * K);
            const double c = double(Q * R) + 0.5 * reads;
            if (c < bc) {
                bc = c;
                best = Tile{R, Q, n};
            }
        }
    return best;
}

// LDS geometry of a group of P planes.  Level 0 holds the input planes,
// level l >= 1 the four subbands of each plane.  Arrays are padded to whole
// tiles and carry a zero border of p = k/2; pitches are odd so that the lanes
// of a wavefront, which read tiles R columns and Q rows apart, spread over
// the LDS banks.  The weight-gradient kernel adds compact, border-free copies
// of levels 1..L for the analysis of dy.
template <int K_, int L_, int H_, int W_, int P_, int NT_>
struct Geo {
    static constexpr int K = K_, L = L_, H = H_, W = W_, P = P_, NT = NT_;
    static constexpr int p = K / 2, KK = K * K;
    static constexpr Tile TL = plan_tile(K, L, H, W, P, NT, 32);
    static constexpr int R = TL.R, Q = TL.Q, NJ = TL.jobs;
    static_assert(R > 0 && NJ <= NT, "no tile fits one job per lane");
    __host__ __device__ static constexpr int hl(int l) { return H >> l; }
    __host__ __device__ static constexpr int wl(int l) { return W >> l; }
    __host__ __device__ static constexpr int S(int l) { return l ? 4 : 1; }
    __host__ __device__ static constexpr int NS(int l) { return cdiv(wl(l), R); }
    __host__ __device__ static constexpr int NG(int l) { return cdiv(hl(l), Q); }
    __host__ __device__ static constexpr int jobs(int l) { return P * S(l) * NS(l) * NG(l); }
    __host__ __device__ static constexpr int jstart(int l) {
        int n = 0;
        for (int m = 0; m < l; ++m) n += jobs(m);
        return n;
    }
    __host__ __device__ static constexpr int rows(int l) { return NG(l) * Q + 2 * p; }
    __host__ __device__ static constexpr int pitch(int l) { return (NS(l) * R + 2 * p) | 1; }
    __host__ __device__ static constexpr int arr(int l) { return rows(l) * pitch(l); }
    __host__ __device__ static constexpr int off(int l) {
        int o = 0;
        for (int m = 0; m < l; ++m) o += P * S(m) * arr(m);
        return o;
    }
    static constexpr int side = off(L + 1);
    // compact dy-side arrays, levels 1..L
    __host__ __device__ static constexpr int vpitch(int l) { return NS(l) * R; }
    __host__ __device__ static constexpr int varr(int l) { return NG(l) * Q * vpitch(l); }
    __host__ __device__ static constexpr int voff(int l) {
        int o = side;
        for (int m = 1; m < l; ++m) o += P * 4 * varr(m);
        return o;
    }
    static constexpr int vside = voff(L + 1) - side;
    static constexpr int NWF = KK * (1 + 4 * L) + 1;  // folded filters + bias
    static constexpr int NPART = KK + 1 + 4 * L * KK; // weight-gradient row
    // element (i, j) of x-side array (level l, plane pl, subband s); i and j
    // may reach into the border
    __host__ __device__ static constexpr int uidx(int l, int pl, int s, int i, int j) {
        return off(l) + (pl * S(l) + s) * arr(l) + (i + p) * pitch(l) + p + j;
    }
    __host__ __device__ static constexpr int vidx(int l, int pl, int s, int i, int j) {
        return voff(l) + (pl * 4 + s) * varr(l) + i * vpitch(l) + j;
    }
    static_assert((H % (1 << L)) == 0 && (W % (1 << L)) == 0, "H, W % 2^L");
    static_assert(NT % 64 == 0, "whole waves");
};

// One lane's tile: array level, plane, subband, tile row group and column
// strip.  Decoded once; the lane keeps it on every group of planes.
struct Job {
    int lvl, pl, s, grp, strip;
    bool on;
};

template <class G>
__device__ __forceinline__ Job decode_job(int t) {
    Job j{0, 0, 0, 0, 0, t < G::NJ};
    static_for<0, G::L + 1>([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        if (t >= G::jstart(l) && t < G::jstart(l + 1)) {
            int r = t - G::jstart(l);
            j.lvl = l;
            j.strip = r % G::NS(l);
            r /= G::NS(l);
            j.grp = r % G::NG(l);
            r /= G::NG(l);
            j.s = r % G::S(l);
            j.pl = r / G::S(l);
        }
    });
    return j;
}

// Per-level constants picked at run time by the lane's level.
template <class G, class F>
__device__ __forceinline__ int by_level(int lvl, F f) {
    int v = f(std::integral_constant<int, 0>{});
    static_for<1, G::L + 1>([&](auto lc) {
        if (lvl == decltype(lc)::value) v = f(lc);
    });
    return v;
}

// ---------------------------------------------------------------------------
// Vector memory helpers
// ---------------------------------------------------------------------------

template <typename T>
constexpr int vec_elems(int n) {
    int v = 16 / int(sizeof(T));
    while (v > 1 && (n % v)) v /= 2;
    return v;
}

template <typename T, int V>
__device__ __forceinline__ void load_vec(const T* __restrict__ src, float (&v)[V]) {
    if constexpr (std::is_same<T, float>::value && V == 4) {
        const float4 q = *reinterpret_cast<const float4*>(src);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else if constexpr (std::is_same<T, float>::value && V == 2) {
        const float2 q = *reinterpret_cast<const float2*>(src);
        v[0] = q.x; v[1] = q.y;
    } else if constexpr (std::is_same<T, __half>::value && V == 8) {
        union { uint4 u; __half2 h[4]; } pk;
        pk.u = *reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float2 f = __half22float2(pk.h[e]);
            v[2 * e] = f.x;
            v[2 * e + 1] = f.y;
        }
    } else if constexpr (std::is_same<T, __half>::value && V == 4) {
        union { uint2 u; __half2 h[2]; } pk;
        pk.u = *reinterpret_cast<const uint2*>(src);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float2 f = __half22float2(pk.h[e]);
            v[2 * e] = f.x;
            v[2 * e + 1] = f.y;
        }
    } else if constexpr (std::is_same<T, __half>::value && V == 2) {
        const float2 f = __half22float2(*reinterpret_cast<const __half2*>(src));
        v[0] = f.x;
        v[1] = f.y;
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = to_f(src[e]);
    }
}

template <typename T, int V>
__device__ __forceinline__ void store_vec(T* __restrict__ dst, const float (&v)[V]) {
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

// HBM -> LDS for planes b0..b0+P-1 (zeros past B), two rows by V columns per
// item, with the level-1 butterflies of those 2 x V pixels computed from the
// same registers.  WRITE_X stores the pixels themselves (x side); the level-1
// subbands go to the x side (U) or the compact dy side (V).
template <class G, typename T, bool WRITE_X, bool VSIDE>
__device__ __forceinline__ void load_level1(float* lds, const T* __restrict__ src, int b0,
                                            int B, int C, int c, int tid) {
    constexpr int V = vec_elems<T>(G::W);
    static_assert(V % 2 == 0, "even column groups");
    constexpr int NV = G::W / V, RP = G::H / 2;
    constexpr int ITEMS = G::P * RP * NV;
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int cv = item % NV;
            const int rp = (item / NV) % RP;
            const int pl = item / (NV * RP);
            const int b = b0 + pl;
            float a[V], d[V];
            if (b < B) {
                const T* s = src + ((size_t(b) * C + c) * G::H + 2 * rp) * G::W + cv * V;
                load_vec<T, V>(s, a);
                load_vec<T, V>(s + G::W, d);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) a[e] = d[e] = 0.f;
            }
            if constexpr (WRITE_X) {
                float* x0 = lds + G::uidx(0, pl, 0, 2 * rp, cv * V);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    x0[e] = a[e];
                    x0[G::pitch(0) + e] = d[e];
                }
            }
#pragma unroll
            for (int m = 0; m < V / 2; ++m) {
                const float p0 = a[2 * m], p1 = a[2 * m + 1], q0 = d[2 * m], q1 = d[2 * m + 1];
                const float s0 = p0 + p1, d0 = p0 - p1, s1 = q0 + q1, d1 = q0 - q1;
                const int j = cv * (V / 2) + m;
                if constexpr (VSIDE) {
                    float* o = lds + G::vidx(1, pl, 0, rp, j);
                    constexpr int A = G::varr(1);
                    o[0] = s0 + s1;
                    o[A] = d0 + d1;
                    o[2 * A] = s0 - s1;
                    o[3 * A] = d0 - d1;
                } else {
                    float* o = lds + G::uidx(1, pl, 0, rp, j);
                    constexpr int A = G::arr(1);
                    o[0] = s0 + s1;
                    o[A] = d0 + d1;
                    o[2 * A] = s0 - s1;
                    o[3 * A] = d0 - d1;
                }
            }
        }
    }
}

// Level-l analysis (l >= 2) from the raw LL of level l-1:
// (a, b; c, d) -> LL = a+b+c+d, LH = a-b+c-d, HL = a+b-c-d, HH = a-b-c+d.
template <class G, int l, bool VSIDE>
__device__ __forceinline__ void analysis_level(float* lds, int tid) {
    constexpr int h = G::hl(l), w = G::wl(l), ITEMS = G::P * h * w;
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int j = item % w;
            const int i = (item / w) % h;
            const int pl = item / (w * h);
            const float* s;
            int sp;
            float* o;
            int A;
            if constexpr (VSIDE) {
                s = lds + G::vidx(l - 1, pl, 0, 2 * i, 2 * j);
                sp = G::vpitch(l - 1);
                o = lds + G::vidx(l, pl, 0, i, j);
                A = G::varr(l);
            } else {
                s = lds + G::uidx(l - 1, pl, 0, 2 * i, 2 * j);
                sp = G::pitch(l - 1);
                o = lds + G::uidx(l, pl, 0, i, j);
                A = G::arr(l);
            }
            const float a = s[0], b = s[1], c = s[sp], d = s[sp + 1];
            const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
            o[0] = s0 + s1;
            o[A] = d0 + d1;
            o[2 * A] = s0 - s1;
            o[3 * A] = d0 - d1;
        }
    }
}

// Top-left element of the conv window of the lane's tile (x side).
template <class G>
__device__ __forceinline__ int window_index(const Job& j) {
    return by_level<G>(j.lvl, [&](auto lc) {
        constexpr int l = decltype(lc)::value;
        return G::uidx(l, j.pl, j.s, j.grp * G::Q - G::p, j.strip * G::R - G::p);
    });
}

template <class G>
__device__ __forceinline__ int level_pitch(int lvl) {
    return by_level<G>(lvl, [&](auto lc) { return G::pitch(decltype(lc)::value); });
}

// acc[q][j] = sum_{u,v} w[u*K+v] * src[(q+u)*pitch + j+v].
template <int K, int Q, int R>
__device__ __forceinline__ void conv_tile(const float* src, int pitch, const float (&w)[K * K],
                                          float (&acc)[Q][R]) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[q][j] = 0.f;
#pragma unroll
    for (int ir = 0; ir < Q + K - 1; ++ir) {
        float in[R + K - 1];
        const float* row = src + ir * pitch;
#pragma unroll
        for (int m = 0; m < R + K - 1; ++m) in[m] = row[m];
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

// acc[u*K+v] += sum_{q,j} d[q][j] * src[(q+u)*pitch + j+v].
template <int K, int Q, int R>
__device__ __forceinline__ void corr_tile(const float (&d)[Q][R], const float* src, int pitch,
                                          float (&acc)[K * K]) {
#pragma unroll
    for (int ir = 0; ir < Q + K - 1; ++ir) {
        float in[R + K - 1];
        const float* row = src + ir * pitch;
#pragma unroll
        for (int m = 0; m < R + K - 1; ++m) in[m] = row[m];
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

// Fold level l's convolved subbands into the LL of level l-1.  A coarse
// coefficient lands on the 2x2 block below it with the sign its subband has
// at each position: the column bit flips LH and HH, the row bit HL and HH.
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
            const float* cs = lds + G::uidx(l, pl, 0, i >> 1, j >> 1);
            const float sy = (i & 1) ? -1.f : 1.f, sx = (j & 1) ? -1.f : 1.f;
            const float e = fmaf(sy, cs[2 * A], cs[0]);
            const float f = fmaf(sy, cs[3 * A], cs[A]);
            lds[G::uidx(l - 1, pl, 0, i, j)] += fmaf(sx, f, e);
        }
    }
}

// y = base conv (already in the level-0 array) + bias + level-1 synthesis,
// V output columns per item, vector store to HBM.
template <class G, typename T>
__device__ __forceinline__ void final_out(const float* lds, float bias, T* __restrict__ out,
                                          int b0, int B, int C, int c, int tid) {
    constexpr int V = vec_elems<T>(G::W);
    constexpr int NV = G::W / V, ITEMS = G::P * G::H * NV;
    constexpr int A1 = G::arr(1);
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int cv = item % NV;
            const int y = (item / NV) % G::H;
            const int pl = item / (NV * G::H);
            const float sy = (y & 1) ? -1.f : 1.f;
            const float* xb = lds + G::uidx(0, pl, 0, y, cv * V);
            const float* cs = lds + G::uidx(1, pl, 0, y >> 1, cv * (V / 2));
            float v[V];
#pragma unroll
            for (int m = 0; m < V / 2; ++m) {
                const float e = fmaf(sy, cs[2 * A1 + m], cs[m]);
                const float f = fmaf(sy, cs[3 * A1 + m], cs[A1 + m]);
                v[2 * m] = xb[2 * m] + bias + (e + f);
                v[2 * m + 1] = xb[2 * m + 1] + bias + (e - f);
            }
            const int b = b0 + pl;
            if (b < B) store_vec<T, V>(out + ((size_t(b) * C + c) * G::H + y) * G::W + cv * V, v);
        }
    }
}

// Folded filters into LDS: [0, KK) base, then (l, s) blocks, then the bias.
template <class G, typename T, bool FLIP>
__device__ __forceinline__ void fold_weights(float* wf, const T* __restrict__ wb,
                                             const T* __restrict__ bb, const T* __restrict__ sb,
                                             const T* __restrict__ ww, const T* __restrict__ sw,
                                             int C, int c, int tid) {
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

// Forward (FLIP = false) or input gradient (FLIP = true) for channel
// blockIdx.x % C over `gpw` groups of P planes starting at group
// (blockIdx.x / C) * gpw.
template <int K, int L, int H, int W, int P, int NT, typename T, bool FLIP>
__global__ __launch_bounds__(NT) void k_plane_apply(
    const T* __restrict__ in, const T* __restrict__ wb, const T* __restrict__ bb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    T* __restrict__ out, int B, int C, int gpw) {
    using G = Geo<K, L, H, W, P, NT>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    float* wf = lds + G::side;
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    for (int i = tid; i < G::side; i += NT) lds[i] = 0.f;
    fold_weights<G, T, FLIP>(wf, wb, bb, sb, ww, sw, C, c, tid);
    __syncthreads();

    const Job job = decode_job<G>(tid);
    const int wsrc = job.lvl == 0 ? 0 : KK * (1 + (job.lvl - 1) * 4 + job.s);
    float w[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) w[t] = wf[wsrc + t];
    const float bias = wf[G::NWF - 1];
    const int win = window_index<G>(job);
    const int pitch = level_pitch<G>(job.lvl);
    const int hrows = by_level<G>(job.lvl, [](auto lc) { return G::hl(decltype(lc)::value); });
    const int wcols = by_level<G>(job.lvl, [](auto lc) { return G::wl(decltype(lc)::value); });
    const int nrows = min(Q, hrows - job.grp * Q);
    const int ncols = min(R, wcols - job.strip * R);
    const int dst = win + G::p * pitch + G::p;  // tile's first output element

    const int ngroups = cdiv(B, P);
    const int g0 = chunk * gpw;
    const int g1 = min(g0 + gpw, ngroups);
    for (int g = g0; g < g1; ++g) {
        const int b0 = g * P;
        load_level1<G, T, true, false>(lds, in, b0, B, C, c, tid);
        __syncthreads();
        static_for<2, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            __syncthreads();
        });
        float acc[Q][R];
        if (job.on) conv_tile<K, Q, R>(lds + win, pitch, w, acc);
        __syncthreads();
        if (job.on) {
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int j = 0; j < R; ++j)
                    if (q < nrows && j < ncols) lds[dst + q * pitch + j] = acc[q][j];
        }
        __syncthreads();
        static_for<0, L - 1>([&](auto lc) {
            cascade_level<G, L - decltype(lc)::value>(lds, tid);
            __syncthreads();
        });
        final_out<G, T>(lds, bias, out, b0, B, C, c, tid);
        __syncthreads();
    }
}

// Weight-gradient partial sums of channel blockIdx.x % C over the groups of
// chunk blockIdx.x / C: one row of G::NPART floats per workgroup,
// [G_b (KK), sum dy, G[l][s] (4 L KK)].
template <int K, int L, int H, int W, int P, int NT, typename T>
__global__ __launch_bounds__(NT) void k_plane_bww(const T* __restrict__ x,
                                                  const T* __restrict__ dy,
                                                  float* __restrict__ part, int B, int C,
                                                  int gpw) {
    using G = Geo<K, L, H, W, P, NT>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    for (int i = tid; i < G::side + G::vside; i += NT) lds[i] = 0.f;
    __syncthreads();

    const Job job = decode_job<G>(tid);
    const int win = window_index<G>(job);
    const int pitch = level_pitch<G>(job.lvl);
    const int hrows = by_level<G>(job.lvl, [](auto lc) { return G::hl(decltype(lc)::value); });
    const int wcols = by_level<G>(job.lvl, [](auto lc) { return G::wl(decltype(lc)::value); });
    const int nrows = min(Q, hrows - job.grp * Q);
    const int ncols = min(R, wcols - job.strip * R);
    const int vsrc = by_level<G>(job.lvl, [&](auto lc) {
        constexpr int l = decltype(lc)::value;
        if constexpr (l == 0) return 0;
        else return G::vidx(l, job.pl, job.s, job.grp * Q, job.strip * R);
    });
    const int vp = by_level<G>(job.lvl, [](auto lc) {
        constexpr int l = decltype(lc)::value;
        if constexpr (l == 0) return 0;
        else return G::vpitch(l);
    });

    float acc[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[t] = 0.f;
    float sdy = 0.f;

    const int ngroups = cdiv(B, P);
    const int g0 = chunk * gpw;
    const int g1 = min(g0 + gpw, ngroups);
    for (int g = g0; g < g1; ++g) {
        const int b0 = g * P;
        load_level1<G, T, true, false>(lds, x, b0, B, C, c, tid);
        load_level1<G, T, false, true>(lds, dy, b0, B, C, c, tid);
        __syncthreads();
        static_for<2, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            analysis_level<G, decltype(lc)::value, true>(lds, tid);
            __syncthreads();
        });
        if (job.on) {
            float d[Q][R];
            if (job.lvl == 0) {
                // base taps: dy straight from HBM (the tile's own pixels)
                // addresses are clamped into the tensor; padding reads as 0
                const int b = b0 + job.pl;
                const T* dp = dy + (size_t(min(b, B - 1)) * C + c) * H * W;
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        const bool ok = b < B && q < nrows && j < ncols;
                        const int yy = min(job.grp * Q + q, H - 1);
                        const int xx = min(job.strip * R + j, W - 1);
                        const float v = to_f(dp[yy * W + xx]);
                        d[q][j] = ok ? v : 0.f;
                        sdy += d[q][j];
                    }
            } else {
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int j = 0; j < R; ++j) d[q][j] = lds[vsrc + q * vp + j];
            }
            corr_tile<K, Q, R>(d, lds + win, pitch, acc);
        }
        __syncthreads();
    }

    // fixed-order workgroup reduction: lane sums of each (array, subband)
    float* red = lds;  // [NT][KK + 1]
    constexpr int RS = KK + 1;
#pragma unroll
    for (int t = 0; t < KK; ++t) red[tid * RS + t] = acc[t];
    red[tid * RS + KK] = sdy;
    __syncthreads();
    for (int o = tid; o < G::NPART; o += NT) {
        float s = 0.f;
        if (o <= KK) {
            for (int t = G::jstart(0); t < G::jstart(1); ++t) s += red[t * RS + o];
        } else {
            const int r = o - KK - 1, ls = r / KK, tap = r % KK;
            const int l = (ls >> 2) + 1, sb = ls & 3;
            by_level<G>(l, [&](auto lc) {
                constexpr int lv = decltype(lc)::value;
                if constexpr (lv > 0) {
                    constexpr int per = G::NS(lv) * G::NG(lv);
                    for (int pl = 0; pl < P; ++pl) {
                        const int t0 = G::jstart(lv) + (pl * 4 + sb) * per;
                        for (int t = t0; t < t0 + per; ++t) s += red[t * RS + tap];
                    }
                }
                return 0;
            });
        }
        part[(size_t(chunk) * C + c) * G::NPART + o] = s;
    }
}

// Sum the partial rows of every chunk in order and apply the chain rule
// through the fold: dKb = beta G_b, dbias = beta sum dy,
// dbeta = <Kb, G_b> + bias sum dy, dK[l,s] = gamma 4^-l G[l,s],
// dgamma[l,s] = 4^-l <K[l,s], G[l,s]>.  nchunk = 0 gives zero gradients.
template <typename T>
__global__ __launch_bounds__(256) void k_bww_final(
    const float* __restrict__ part, int nchunk, int C, int K, int L, const T* __restrict__ wb,
    const T* __restrict__ bb, const T* __restrict__ sb, const T* __restrict__ ww,
    const T* __restrict__ sw, T* __restrict__ dwb, T* __restrict__ dbb, T* __restrict__ dsb,
    T* __restrict__ dww, T* __restrict__ dsw) {
    extern __shared__ float g[];
    const int KK = K * K, NPART = KK + 1 + 4 * L * KK;
    const int c = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    for (int i = tid; i < NPART; i += nt) {
        float v[8];
        float s = 0.f;
        for (int ch0 = 0; ch0 < nchunk; ch0 += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = ch0 + u < nchunk ? part[(size_t(ch0 + u) * C + c) * NPART + i] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
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
    const size_t la = sizeof(float) * (G::side + G::NWF);
    size_t lb = sizeof(float) * (G::side + G::vside);
    const size_t lr = sizeof(float) * NT * (G::KK + 1);
    if (lb < lr) lb = lr;
    return Variant{K, L, H, W, dtype, P, NT,
                   reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, false>),
                   reinterpret_cast<const void*>(&k_plane_apply<K, L, H, W, P, NT, T, true>),
                   reinterpret_cast<const void*>(&k_plane_bww<K, L, H, W, P, NT, T>),
                   la, lb};
}

// (K, L, H, W, planes per group, threads).  The ConvNeXt-T stage shapes
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
    X(5, 6, 64, 64, 1, 512)

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

// Groups of planes per workgroup: enough workgroups to cover the chip about
// three times, each walking a contiguous run of groups of one channel.
int groups_per_wg(const wtconv_shape& s, int P) {
    const int ngroups = cdiv(s.B, P);
    const long total = long(ngroups) * s.C;
    const long target = 768;
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
    const int gpw = groups_per_wg(s, v->P);
    const int nchunk = cdiv(cdiv(s.B, v->P), gpw);
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
    int gpw = groups_per_wg(s, v->P), B = s.B, C = s.C;
    const int nchunk = cdiv(cdiv(s.B, v->P), gpw);
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

hipError_t plane_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                            const Params& p, const Grads& g, void* workspace,
                            hipStream_t stream) {
    const Variant* v = find_variant(s);
    if (!v) return hipErrorInvalidValue;
    hipError_t e = prepare(v->bww, v->lds_bww);
    if (e != hipSuccess) return e;
    int gpw = groups_per_wg(s, v->P), B = s.B, C = s.C;
    const int nchunk = cdiv(cdiv(s.B, v->P), gpw);
    float* part = static_cast<float*>(workspace);
    void* args[] = {&x, &dy, &part, &B, &C, &gpw};
    e = hipLaunchKernel(v->bww, dim3(unsigned(nchunk) * unsigned(s.C)), dim3(v->NT), args,
                        v->lds_bww, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, part, nchunk, p, g, stream)
                                 : launch_final<__half>(s, part, nchunk, p, g, stream);
}

hipError_t zero_grads(const wtconv_shape& s, const Params& p, const Grads& g,
                      hipStream_t stream) {
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, nullptr, 0, p, g, stream)
                                 : launch_final<__half>(s, nullptr, 0, p, g, stream);
}

}  // namespace wtc
