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
            const double c = double(Q * R) + 0.5 * reads + ((R & 1) ? 0.0 : 0.01);
            if (c < bc) {
                bc = c;
                best = Tile{R, Q, n};
            }
        }
    return best;
}

// LDS layout of one level: row pitch, stride between the 2-D arrays of the
// level (one per plane and subband) and the level's start offset.
struct Layout {
    int pitch, astride, off;
};

// Bank multiplicity of the tiles' window reads: for every 32 consecutive
// lanes (the lanes that share an LDS cycle), the most lanes that hit one of
// 32 four-byte banks, summed over the level's lanes.  Every read of a tile is
// its window address plus the same constant, so window addresses decide.
constexpr int bank_cost(int first_job, int njobs_l, int S, int NS, int NG, int R, int Q,
                        int pitch, int astride, int off) {
    int cost = 0;
    const int n0 = first_job & ~31, n1 = first_job + njobs_l;
    for (int w = n0; w < n1; w += 32) {
        int cnt[32] = {};
        int mx = 0;
        for (int n = w; n < w + 32 && n < n1; ++n) {
            if (n < first_job) continue;
            int r = n - first_job;
            const int strip = r % NS;
            r /= NS;
            const int grp = r % NG;
            const int ps = r / NG;  // plane * S + subband
            const int a = off + ps * astride + grp * Q * pitch + strip * R;
            const int b = ((a % 32) + 32) % 32;
            if (++cnt[b] > mx) mx = cnt[b];
        }
        cost += mx;
    }
    (void)S;
    return cost;
}

// Level start, pitch and array gap, each over one period of the bank index:
// the level starts on the bank of its first lane's tile (R times its job
// index), then the pitch is searched with no gap, then the gap.  Least bank
// multiplicity wins, then least LDS.
constexpr Layout plan_layout(int first_job, int njobs_l, int S, int NS, int NG, int R, int Q,
                             int rows, int minpitch, int base) {
    int off = base;
    while (((off - R * first_job) % 32 + 32) % 32 != 0) ++off;
    int bp = minpitch, bc = 1 << 30;
    for (int dp = 0; dp < 32; ++dp) {
        const int c = bank_cost(first_job, njobs_l, S, NS, NG, R, Q, minpitch + dp,
                                rows * (minpitch + dp), off);
        if (c < bc) {
            bc = c;
            bp = minpitch + dp;
        }
    }
    int bg = 0;
    bc = 1 << 30;
    for (int gap = 0; gap < 32; ++gap) {
        const int c = bank_cost(first_job, njobs_l, S, NS, NG, R, Q, bp, rows * bp + gap, off);
        if (c < bc) {
            bc = c;
            bg = gap;
        }
    }
    return Layout{bp, rows * bp + bg, off};
}

// LDS geometry of a group of P planes.  Level 0 holds the input planes,
// level l >= 1 the four subbands of each plane.  Arrays are padded to whole
// tiles and carry a zero border of p = k/2; pitches and gaps are searched so
// that the lanes of a wavefront, each reading its own tile window, spread
// over the LDS banks.  The weight-gradient kernel adds compact, border-free
// copies of levels 1..L for the analysis of dy.
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

    struct Table {
        Layout lv[L_ + 1];
        int end;
    };
    static constexpr Table make_table() {
        Table t{};
        int base = 0;
        for (int l = 0; l <= L; ++l) {
            t.lv[l] = plan_layout(jstart(l), jobs(l), S(l), NS(l), NG(l), R, Q, rows(l),
                                  NS(l) * R + 2 * p, base);
            base = t.lv[l].off + P * S(l) * t.lv[l].astride;
        }
        t.end = base;
        return t;
    }
    static constexpr Table TB = make_table();
    __host__ __device__ static constexpr int pitch(int l) { return TB.lv[l].pitch; }
    __host__ __device__ static constexpr int arr(int l) { return TB.lv[l].astride; }
    __host__ __device__ static constexpr int off(int l) { return TB.lv[l].off; }
    static constexpr int side = TB.end;
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

template <int BYTES>
struct RawVec;
template <>
struct RawVec<16> { using type = uint4; };
template <>
struct RawVec<8> { using type = uint2; };
template <>
struct RawVec<4> { using type = uint32_t; };

// One thread's share of a group's input, held as the raw bytes loaded from
// HBM so that the loads can be issued a whole group ahead of their use.  An
// item is ROWS rows by V columns: with four rows the level-2 butterflies are
// computed from registers too.
template <class G, typename T>
struct Fetch {
    static constexpr int V = vec_elems<T>(G::W);
    static_assert(V % 2 == 0, "even column groups");
    static constexpr int ROWS = (G::L >= 2 && V % 4 == 0) ? 4 : 2;
    static constexpr int NV = G::W / V, RB = G::H / ROWS;
    static constexpr int ITEMS = G::P * RB * NV, IT = cdiv(ITEMS, G::NT);
    static constexpr int LEVELS = ROWS == 4 ? 2 : 1;  // levels computed here
    using raw_t = typename RawVec<V * int(sizeof(T))>::type;
    raw_t r[IT][ROWS];

    // Issue the loads of planes b0..b0+P-1 (zeros past B).
    __device__ __forceinline__ void issue(const T* __restrict__ src, int b0, int B, int C,
                                          int c, int tid) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int item = tid + it * G::NT;
            const int cv = item % NV;
            const int rb = (item / NV) % RB;
            const int pl = item / (NV * RB);
            const int b = b0 + pl;
            if ((ITEMS % G::NT == 0 || item < ITEMS) && b < B) {
                const raw_t* s = reinterpret_cast<const raw_t*>(
                    src + ((size_t(b) * C + c) * G::H + ROWS * rb) * G::W + cv * V);
#pragma unroll
                for (int k = 0; k < ROWS; ++k) r[it][k] = s[k * (G::W / V)];
            } else {
#pragma unroll
                for (int k = 0; k < ROWS; ++k) r[it][k] = raw_t{};
            }
        }
    }

    static __device__ __forceinline__ void unpack(const raw_t& raw, float (&v)[V]) {
        union {
            raw_t r;
            T e[V];
        } u;
        u.r = raw;
#pragma unroll
        for (int k = 0; k < V; ++k) v[k] = to_f(u.e[k]);
    }

    // (a, b; c, d) -> LL, LH, HL, HH of one 2x2 block, unnormalised.
    static __device__ __forceinline__ void butterfly(float a, float b, float c, float d,
                                                     float (&o)[4]) {
        const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
        o[0] = s0 + s1;
        o[1] = d0 + d1;
        o[2] = s0 - s1;
        o[3] = d0 - d1;
    }

    template <bool VSIDE>
    static __device__ __forceinline__ void put(float* lds, int l, int pl, int i, int j,
                                               const float (&o)[4]) {
        float* dst;
        int A;
        if constexpr (VSIDE) {
            dst = lds + G::vidx(l, pl, 0, i, j);
            A = l == 1 ? G::varr(1) : G::varr(2);
        } else {
            dst = lds + G::uidx(l, pl, 0, i, j);
            A = l == 1 ? G::arr(1) : G::arr(G::L >= 2 ? 2 : 1);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) dst[s * A] = o[s];
    }

    // Write the pixels to the level-0 array (WRITE_X) and the level-1 (and,
    // with four-row items, level-2) butterflies to the x side or the dy side.
    template <bool WRITE_X, bool VSIDE>
    __device__ __forceinline__ void commit(float* lds, int tid) const {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int item = tid + it * G::NT;
            if (ITEMS % G::NT == 0 || item < ITEMS) {
                const int cv = item % NV;
                const int rb = (item / NV) % RB;
                const int pl = item / (NV * RB);
                float x[ROWS][V];
#pragma unroll
                for (int k = 0; k < ROWS; ++k) unpack(r[it][k], x[k]);
                if constexpr (WRITE_X) {
                    float* o = lds + G::uidx(0, pl, 0, ROWS * rb, cv * V);
#pragma unroll
                    for (int k = 0; k < ROWS; ++k)
#pragma unroll
                        for (int e = 0; e < V; ++e) o[k * G::pitch(0) + e] = x[k][e];
                }
                float ll[ROWS / 2][V / 2];
#pragma unroll
                for (int rr = 0; rr < ROWS / 2; ++rr)
#pragma unroll
                    for (int m = 0; m < V / 2; ++m) {
                        float o[4];
                        butterfly(x[2 * rr][2 * m], x[2 * rr][2 * m + 1], x[2 * rr + 1][2 * m],
                                  x[2 * rr + 1][2 * m + 1], o);
                        ll[rr][m] = o[0];
                        put<VSIDE>(lds, 1, pl, (ROWS / 2) * rb + rr, cv * (V / 2) + m, o);
                    }
                if constexpr (ROWS == 4) {
#pragma unroll
                    for (int m = 0; m < V / 4; ++m) {
                        float o[4];
                        butterfly(ll[0][2 * m], ll[0][2 * m + 1], ll[1][2 * m], ll[1][2 * m + 1], o);
                        put<VSIDE>(lds, 2, pl, rb, cv * (V / 4) + m, o);
                    }
                }
            }
        }
    }
};

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
                                          float init, float (&acc)[Q][R]) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[q][j] = init;
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

// y = base conv plus bias (already in the level-0 array) + synthesis, written
// back in place.  Each item covers two output rows (one level-1 coefficient
// row) by V columns.  Level 2, whose coarser levels are already folded into
// its LL, is folded into the level-1 LL here, on the fly; then each level-1
// coefficient is expanded over its 2x2 block.
template <class G, typename T>
__device__ __forceinline__ void final_to_lds(float* lds, int tid) {
    constexpr int V = vec_elems<T>(G::W);
    constexpr int NV = G::W / V, RP = G::H / 2, ITEMS = G::P * RP * NV;
    constexpr int A1 = G::arr(1);
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int cv = item % NV;
            const int i = (item / NV) % RP;
            const int pl = item / (NV * RP);
            float* x0 = lds + G::uidx(0, pl, 0, 2 * i, cv * V);
            const float* cs = lds + G::uidx(1, pl, 0, i, cv * (V / 2));
#pragma unroll
            for (int m = 0; m < V / 2; ++m) {
                float ll = cs[m];
                if constexpr (G::L >= 2) {
                    constexpr int A2 = G::arr(2);
                    const int j = cv * (V / 2) + m;
                    const float* c2 = lds + G::uidx(2, pl, 0, i >> 1, j >> 1);
                    const float sy2 = (i & 1) ? -1.f : 1.f, sx2 = (j & 1) ? -1.f : 1.f;
                    const float e2 = fmaf(sy2, c2[2 * A2], c2[0]);
                    const float f2 = fmaf(sy2, c2[3 * A2], c2[A2]);
                    ll += fmaf(sx2, f2, e2);
                }
                const float lh = cs[A1 + m], hl = cs[2 * A1 + m], hh = cs[3 * A1 + m];
                const float e0 = ll + hl, f0 = lh + hh;  // row 2i   (row bit 0)
                const float e1 = ll - hl, f1 = lh - hh;  // row 2i+1 (row bit 1)
                x0[2 * m] += e0 + f0;
                x0[2 * m + 1] += e0 - f0;
                x0[G::pitch(0) + 2 * m] += e1 + f1;
                x0[G::pitch(0) + 2 * m + 1] += e1 - f1;
            }
        }
    }
}

// The finished group (y in the level-0 array) -> HBM, ROWS x V per item.
template <class G, typename T>
__device__ __forceinline__ void store_out(const float* lds, T* __restrict__ out, int b0, int B,
                                          int C, int c, int tid) {
    using F = Fetch<G, T>;
    constexpr int V = F::V, ROWS = F::ROWS, NV = F::NV, RB = F::RB, ITEMS = F::ITEMS;
#pragma unroll
    for (int it = 0; it < F::IT; ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int cv = item % NV;
            const int rb = (item / NV) % RB;
            const int pl = item / (NV * RB);
            const int b = b0 + pl;
            if (b < B) {
                const float* x0 = lds + G::uidx(0, pl, 0, ROWS * rb, cv * V);
                T* o = out + ((size_t(b) * C + c) * G::H + ROWS * rb) * G::W + cv * V;
#pragma unroll
                for (int k = 0; k < ROWS; ++k) {
                    float v[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) v[e] = x0[k * G::pitch(0) + e];
                    store_vec<T, V>(o + k * G::W, v);
                }
            }
        }
    }
}

// Wait for every outstanding vector-memory operation (the group's prefetched
// input and stores issued a group earlier).  Stores are then issued only after
// this point, so no later wait for prefetched data has to drain fresh stores.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// Waves per SIMD the LDS footprint allows (NT/64 waves per workgroup spread
// over 4 SIMDs); the register budget is sized to match.
constexpr int waves_for_lds(size_t lds_bytes, int nt) {
    int wg = int(163840 / (lds_bytes ? lds_bytes : 1));
    int w = wg * (nt / 64) / 4;
    return w < 1 ? 1 : (w > 8 ? 8 : w);
}

template <class G>
constexpr size_t apply_lds_bytes() { return sizeof(float) * (G::side + G::NWF); }
template <class G>
constexpr size_t bww_lds_bytes() {
    size_t a = sizeof(float) * (G::side + G::vside), b = sizeof(float) * G::NT * (G::KK + 1);
    return a > b ? a : b;
}

// Forward (FLIP = false) or input gradient (FLIP = true).  The C * ceil(B/P)
// (channel, group of P planes) pairs, channel-major, are split into gridDim.x
// equal contiguous ranges, one per workgroup; the filters are folded again
// whenever a workgroup's range enters a new channel.  The next group's input
// is loaded into registers while the current one is computed, and a group's
// output is stored at the start of the next iteration.
template <int K, int L, int H, int W, int P, int NT, typename T, bool FLIP>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(
    waves_for_lds(apply_lds_bytes<Geo<K, L, H, W, P, NT>>(), NT) < 4
        ? waves_for_lds(apply_lds_bytes<Geo<K, L, H, W, P, NT>>(), NT)
        : 4,
    8))) void k_plane_apply(
    const T* __restrict__ in, const T* __restrict__ wb, const T* __restrict__ bb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    T* __restrict__ out, int B, int C) {
    using G = Geo<K, L, H, W, P, NT>;
    using F = Fetch<G, T>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    float* wf = lds + G::side;
    const int tid = threadIdx.x;
    const int ngroups = cdiv(B, P);
    const long total = long(C) * ngroups;
    const int q0 = int(total * blockIdx.x / gridDim.x);
    const int q1 = int(total * (blockIdx.x + 1) / gridDim.x);
    F fx;
    if (q0 < q1) fx.issue(in, (q0 % ngroups) * P, B, C, q0 / ngroups, tid);
    for (int i = tid; i < G::side; i += NT) lds[i] = 0.f;

    const Job job = decode_job<G>(tid);
    const int wsrc = job.lvl == 0 ? 0 : KK * (1 + (job.lvl - 1) * 4 + job.s);
    const int win = window_index<G>(job);
    const int pitch = level_pitch<G>(job.lvl);
    const int hrows = by_level<G>(job.lvl, [](auto lc) { return G::hl(decltype(lc)::value); });
    const int wcols = by_level<G>(job.lvl, [](auto lc) { return G::wl(decltype(lc)::value); });
    const int nrows = min(Q, hrows - job.grp * Q);
    const int ncols = min(R, wcols - job.strip * R);
    const bool full = nrows == Q && ncols == R;
    const int dst = win + G::p * pitch + G::p;  // tile's first output element

    float w[KK];
    float init = 0.f;
    int cur = -1, pend_b0 = -1, pend_c = 0;
    for (int q = q0; q < q1; ++q) {
        const int c = q / ngroups;
        const int b0 = (q % ngroups) * P;
        if (c != cur) {
            fold_weights<G, T, FLIP>(wf, wb, bb, sb, ww, sw, C, c, tid);
            __syncthreads();
#pragma unroll
            for (int t = 0; t < KK; ++t) w[t] = wf[wsrc + t];
            init = job.lvl == 0 ? wf[G::NWF - 1] : 0.f;
            cur = c;
        }
        wait_vmem();
        if (pend_b0 >= 0) {
            store_out<G, T>(lds, out, pend_b0, B, C, pend_c, tid);
            __syncthreads();
        }
        fx.template commit<true, false>(lds, tid);
        __syncthreads();
        static_for<F::LEVELS + 1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            __syncthreads();
        });
        float acc[Q][R];
        if (job.on) conv_tile<K, Q, R>(lds + win, pitch, w, init, acc);
        // the next group's loads fly during write-back, synthesis and store
        if (q + 1 < q1) fx.issue(in, ((q + 1) % ngroups) * P, B, C, (q + 1) / ngroups, tid);
        __syncthreads();
        if (job.on) {
            if (full) {
#pragma unroll
                for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                    for (int j = 0; j < R; ++j) lds[dst + qq * pitch + j] = acc[qq][j];
            } else {
#pragma unroll
                for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                    for (int j = 0; j < R; ++j)
                        if (qq < nrows && j < ncols) lds[dst + qq * pitch + j] = acc[qq][j];
            }
        }
        __syncthreads();
        // levels L..3 fold into the LL of the level above; level 2 folds into
        // level 1 inside final_to_lds
        static_for<0, L - 2>([&](auto lc) {
            cascade_level<G, L - decltype(lc)::value>(lds, tid);
            __syncthreads();
        });
        final_to_lds<G, T>(lds, tid);
        pend_b0 = b0;
        pend_c = c;
        __syncthreads();
    }
    if (pend_b0 >= 0) store_out<G, T>(lds, out, pend_b0, B, C, pend_c, tid);
}

// Weight-gradient partial sums of channel blockIdx.x % C over the groups of
// chunk blockIdx.x / C: one row of G::NPART floats per workgroup,
// [G_b (KK), sum dy, G[l][s] (4 L KK)].
template <int K, int L, int H, int W, int P, int NT, typename T>
__global__ __launch_bounds__(NT) void k_plane_bww(
    const T* __restrict__ x,
                                                  const T* __restrict__ dy,
                                                  float* __restrict__ part, int B, int C,
                                                  int gpw) {
    using G = Geo<K, L, H, W, P, NT>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    const int ngroups = cdiv(B, P);
    const int g0 = chunk * gpw;
    const int g1 = min(g0 + gpw, ngroups);
    Fetch<G, T> fx, fd;
    fx.issue(x, g0 * P, B, C, c, tid);
    fd.issue(dy, g0 * P, B, C, c, tid);
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

    for (int g = g0; g < g1; ++g) {
        const int b0 = g * P;
        fx.template commit<true, false>(lds, tid);
        fd.template commit<false, true>(lds, tid);
        if (g + 1 < g1) {
            fx.issue(x, b0 + P, B, C, c, tid);
            fd.issue(dy, b0 + P, B, C, c, tid);
        }
        __syncthreads();
        static_for<Fetch<G, T>::LEVELS + 1, L + 1>([&](auto lc) {
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
    const size_t la = apply_lds_bytes<G>();
    const size_t lb = bww_lds_bytes<G>();
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
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, part, nchunk, p, g, stream)
                                 : launch_final<__half>(s, part, nchunk, p, g, stream);
}

hipError_t zero_grads(const wtconv_shape& s, const Params& p, const Grads& g,
                      hipStream_t stream) {
    return s.dtype == WTCONV_F32 ? launch_final<float>(s, nullptr, 0, p, g, stream)
                                 : launch_final<__half>(s, nullptr, 0, p, g, stream);
}

}  // namespace wtc
