// Device code of the fused WTConv kernels for gfx950, shared by the
// translation units that instantiate them (whole planes, tiles, deep levels).
#pragma once
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
//
// The fused backward (input gradient and weight taps in one pass) comes in
// two forms: x and dy side by side in LDS, or -- where a lane's tile is large
// enough -- one set of arrays that x and then dy pass through, with the taps
// taken transposed so that one dy window per tile serves the conv and the
// taps (k_plane_bwd1; on large planes k_tile_bwd1, whose x pass needs only
// the tile's core).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wtconv_internal.h"

namespace wtc {
namespace dev {

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

// Level start, pitch and array gap, each over one period of the bank index.
// The core of every array starts on a multiple of `al` floats and pitch and
// gap keep it there, so that rows can be moved with 8- and 16-byte LDS
// accesses.  Pitch and start are searched together (with al = 1 the start is
// put on the bank of the first lane's tile, R times its job index), then the
// gap.  Least bank multiplicity wins, then least LDS.
constexpr Layout plan_layout(int first_job, int njobs_l, int S, int NS, int NG, int R, int Q,
                             int rows, int minpitch, int base, int h, int al) {
    int p0 = minpitch;
    while (p0 % al) ++p0;
    int bp = p0, boff = base, bc = 1 << 30;
    for (int dp = 0; dp < 32; dp += al) {
        const int pitch = p0 + dp;
        for (int off = base; off < base + 32; ++off) {
            if (al == 1) {
                if (((off - R * first_job) % 32 + 32) % 32 != 0) continue;
            } else if ((off + h * pitch + h) % al != 0) {
                continue;
            }
            const int c = bank_cost(first_job, njobs_l, S, NS, NG, R, Q, pitch, rows * pitch, off);
            if (c < bc) {
                bc = c;
                bp = pitch;
                boff = off;
            }
        }
    }
    int bg = 0;
    bc = 1 << 30;
    for (int gap = 0; gap < 32; gap += al) {
        const int c = bank_cost(first_job, njobs_l, S, NS, NG, R, Q, bp, rows * bp + gap, boff);
        if (c < bc) {
            bc = c;
            bg = gap;
        }
    }
    return Layout{bp, rows * bp + bg, boff};
}

// n consecutive floats between registers and LDS at an element offset that is
// a multiple of A floats (A = 1, 2 or 4): 16-, 8- or 4-byte accesses.
template <int N, int A>
__device__ __forceinline__ void lds_put(float* dst, const float* v) {
    if constexpr (A % 4 == 0 && N % 4 == 0) {
#pragma unroll
        for (int c = 0; c < N; c += 4)
            *reinterpret_cast<float4*>(dst + c) = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
    } else if constexpr (A % 2 == 0 && N % 2 == 0) {
#pragma unroll
        for (int c = 0; c < N; c += 2)
            *reinterpret_cast<float2*>(dst + c) = make_float2(v[c], v[c + 1]);
    } else {
#pragma unroll
        for (int c = 0; c < N; ++c) dst[c] = v[c];
    }
}

template <int N, int A>
__device__ __forceinline__ void lds_get(const float* src, float* v) {
    if constexpr (A % 4 == 0 && N % 4 == 0) {
#pragma unroll
        for (int c = 0; c < N; c += 4) {
            const float4 q = *reinterpret_cast<const float4*>(src + c);
            v[c] = q.x; v[c + 1] = q.y; v[c + 2] = q.z; v[c + 3] = q.w;
        }
    } else if constexpr (A % 2 == 0 && N % 2 == 0) {
#pragma unroll
        for (int c = 0; c < N; c += 2) {
            const float2 q = *reinterpret_cast<const float2*>(src + c);
            v[c] = q.x; v[c + 1] = q.y;
        }
    } else {
#pragma unroll
        for (int c = 0; c < N; ++c) v[c] = src[c];
    }
}

// LDS geometry of a group of P planes.  Level 0 holds the input planes,
// level l >= 1 the four subbands of each plane.  Arrays are padded to whole
// tiles and carry a zero border of p = k/2; pitches and gaps are searched so
// that the lanes of a wavefront, each reading its own tile window, spread
// over the LDS banks.  The weight-gradient kernel adds compact, border-free
// copies of levels 1..L for the analysis of dy.
// HT_ = 0: whole planes (H x W), every array has a zero border of p.
// HT_ > 0: an H x W output tile of a larger plane with HT_ levels handled in
// the tile; level l carries a halo of h(l) = p 2^(HT_-l) real neighbouring
// values (the receptive footprint of the coarser levels) around its core.
// AMAX_ caps the row alignment (floats): 4 lets the row phases use 16-byte
// LDS accesses, 2 leaves the pitch free to spread the conv windows of a
// wavefront over every bank.  TRIM_ (tiles): store less halo on the levels
// the fetch analyses in registers (sh below).
template <int K_, int L_, int H_, int W_, int P_, int NT_, int HT_ = 0, int AMAX_ = 4,
          bool TRIM_ = false>
struct Geo {
    static constexpr int K = K_, L = L_, H = H_, W = W_, P = P_, NT = NT_, HT = HT_;
    static constexpr int p = K / 2, KK = K * K;
    static_assert(HT == 0 || (HT == L && P == 1), "tiles hold one plane, all their levels");
    // receptive halo and the part of it filled with data
    __host__ __device__ static constexpr int h(int l) { return HT ? (p << (HT - l)) : p; }
    __host__ __device__ static constexpr int ah(int l) { return HT ? h(l) : 0; }
    // Levels the halo fetch of a tile analyses in registers (Fetch: four-row
    // items give levels 1 and 2, two-row items level 1).
    __host__ __device__ static constexpr int fetch_levels() {
        return (L >= 2 && ah(0) % 4 == 0 && W % 4 == 0) ? 2 : (L >= 1 ? 1 : 0);
    }
    // Stored halo of level l.  Whole planes: the zero border p.  Tiles: h(l),
    // the footprint of the coarser levels; with TRIM_ only on the levels
    // analysed in LDS (from fetch_levels() on): below those a level is only
    // read by its own conv, so it keeps p, rounded up to the unit the fetch
    // writes it in (8 >> l: four rows by four or eight columns at level 0).
    // The 32 x 64 tile at k = 5 then needs 42.6 KB of LDS instead of 61.6 KB
    // for the forward (41.3 + 1.3 KB for the fused backward), three
    // workgroups per unit instead of two (512^2 forward 619 -> 550 us).
    __host__ __device__ static constexpr int sh(int l) {
        if (!HT || !TRIM_ || l >= fetch_levels()) return h(l);
        const int u = 8 >> l, s = (p + u - 1) / u * u;
        return s < h(l) ? s : h(l);
    }
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
    __host__ __device__ static constexpr int maxi(int a, int b) { return a > b ? a : b; }
    // rows: halo, then the padded core (its last tile's window) or the core
    // plus the far halo, whichever reaches further
    __host__ __device__ static constexpr int rows(int l) {
        return sh(l) + maxi(NG(l) * Q + p, hl(l) + sh(l));
    }
    __host__ __device__ static constexpr int minpitch(int l) {
        return sh(l) + maxi(NS(l) * R + p, wl(l) + sh(l));
    }
    // alignment (floats) of the core rows of level l: the widest LDS access
    // the fp32 item width of the plane (and of the halo) allows, halved per
    // level
    __host__ __device__ static constexpr int vec_f32(int n) {
        return n % 4 == 0 ? 4 : (n % 2 == 0 ? 2 : 1);
    }
    __host__ __device__ static constexpr int al(int l) {
        int a0 = HT ? (vec_f32(W) < vec_f32(ah(0)) ? vec_f32(W) : vec_f32(ah(0))) : vec_f32(W);
        if (a0 > AMAX_) a0 = AMAX_;
        return (a0 >> l) > 1 ? (a0 >> l) : 1;
    }

    struct Table {
        Layout lv[L_ + 1];
        int end;
    };
    static constexpr Table make_table() {
        Table t{};
        int base = 0;
        for (int l = 0; l <= L; ++l) {
            t.lv[l] = plan_layout(jstart(l), jobs(l), S(l), NS(l), NG(l), R, Q, rows(l),
                                  minpitch(l), base, sh(l), al(l));
            base = t.lv[l].off + P * S(l) * t.lv[l].astride;
        }
        t.end = base;
        return t;
    }
    static constexpr Table TB = make_table();
    static constexpr bool aligned_table() {
        for (int l = 0; l <= L; ++l) {
            const int a = al(l), pt = TB.lv[l].pitch, o = TB.lv[l].off;
            if (pt % a || TB.lv[l].astride % a || (o + sh(l) * pt + sh(l)) % a) return false;
        }
        return true;
    }
    static_assert(aligned_table(), "array cores aligned for vector LDS access");
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
        return off(l) + (pl * S(l) + s) * arr(l) + (i + sh(l)) * pitch(l) + sh(l) + j;
    }
    __host__ __device__ static constexpr int vidx(int l, int pl, int s, int i, int j) {
        return voff(l) + (pl * 4 + s) * varr(l) + i * vpitch(l) + j;
    }
    static_assert((H % (1 << L)) == 0 && (W % (1 << L)) == 0, "H, W % 2^L");
    static_assert(NT % 64 == 0, "whole waves");
};

// Layout of the whole-plane gradient kernels: each lane reads two windows
// per tile (dy and x), so window reads outweigh the row phases.
template <int K, int L, int H, int W, int P, int NT>
using GeoGrad = Geo<K, L, H, W, P, NT, 0, 2>;

// Layout of the tile forward and fused backward: trimmed halos below the
// LDS-analysed levels.
template <int K, int LT, int TH, int TW, int NT>
using GeoTileTrim = Geo<K, LT, TH, TW, 1, NT, LT, 4, true>;

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

// Raw buffer resources over one group's planes.  Accesses at or past the
// resource's size read zeros and write nothing, so lanes without an item (or
// planes past the batch) need no branch, and the compiler can count the
// outstanding memory operations of a straight-line loop body exactly.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kBufFlags = 0x00020000;  // raw 32-bit dwords, no swizzle
constexpr int kOutOfRange = int(0x80000000u);  // an offset past every resource here

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufFlags);
}

// Planes b0 .. b0+P-1 of channel c (those below B) of a tensor of HW-element
// planes: base pointer and size.
template <class G, typename T>
struct GroupSpan {
    const T* base;
    int bytes;
    __device__ GroupSpan(const T* src, int b0, int B, int C, int c, int HW = G::H * G::W) {
        const int nvalid = min(G::P, B - b0);
        base = src + (size_t(b0) * C + c) * HW;
        bytes = nvalid > 0 ? ((nvalid - 1) * C * HW + HW) * int(sizeof(T)) : 0;
    }
};

// One element through a buffer resource (offset past the resource: reads
// zero, writes nothing).
template <typename T>
__device__ __forceinline__ T buf_load_elem(rsrc_t r, int off) {
    if constexpr (std::is_same<T, float>::value)
        return __int_as_float(int(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0)));
    else
        return __ushort_as_half(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
template <typename T>
__device__ __forceinline__ void buf_store_elem(T v, rsrc_t r, int off) {
    if constexpr (std::is_same<T, float>::value)
        __builtin_amdgcn_raw_buffer_store_b32(unsigned(__float_as_int(v)), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(__half_as_ushort(v), r, off, 0, 0);
}

template <int BYTES>
__device__ __forceinline__ typename std::conditional<
    BYTES == 16, uint4, typename std::conditional<BYTES == 8, uint2, uint32_t>::type>::type
buf_load(rsrc_t r, int off) {
    if constexpr (BYTES == 16) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        return uint4{v[0], v[1], v[2], v[3]};
    } else if constexpr (BYTES == 8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return uint2{v[0], v[1]};
    } else {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
}

// Buffer stores; AUX is the cache policy (2: non-temporal).
template <int AUX = 0>
__device__ __forceinline__ void buf_store(const uint4& v, rsrc_t r, int off) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(v4u{v.x, v.y, v.z, v.w}, r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store(const uint2& v, rsrc_t r, int off) {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(v2u{v.x, v.y}, r, off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store(const uint32_t& v, rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, AUX);
}

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
template <class G, typename T, bool HALO = (G::HT > 0)>
struct Fetch {
    static constexpr int A0 = HALO ? G::ah(0) : 0;  // halo loaded around the core
    static constexpr int V = HALO ? (vec_elems<T>(G::W) < vec_elems<T>(A0) ? vec_elems<T>(G::W)
                                                                            : vec_elems<T>(A0))
                                  : vec_elems<T>(G::W);
    static_assert(V % 2 == 0, "even column groups");
    static constexpr int ROWS = (G::L >= 2 && V % 4 == 0 && (A0 % 4) == 0) ? 4 : 2;
    static constexpr int FH = G::H + 2 * A0, FW = G::W + 2 * A0;
    static constexpr int NV = FW / V, RB = FH / ROWS;
    static_assert(FW % V == 0 && FH % ROWS == 0, "footprint in whole items");
    static constexpr int ITEMS = G::P * RB * NV, IT = cdiv(ITEMS, G::NT);
    static constexpr int LEVELS = ROWS == 4 ? 2 : (G::L >= 1 ? 1 : 0);  // levels computed here
    static_assert(!HALO || LEVELS == G::fetch_levels(), "the layout's view of the fetch");
    // a level-l item (ROWS >> l rows, V >> l columns, placed at -A0 >> l plus
    // whole items) lies entirely inside or entirely outside the stored halo
    static constexpr bool whole_items() {
        for (int l = 0; l < LEVELS && l < 2; ++l) {
            const int d = (A0 >> l) - G::sh(l), nr = ROWS >> l, nc = V >> l;
            if (d < 0 || (nr && d % nr) || (nc && d % nc)) return false;
        }
        return true;
    }
    static_assert(!HALO || whole_items(), "fetch items straddle the stored halo");
    using raw_t = typename RawVec<V * int(sizeof(T))>::type;
    raw_t r[IT][ROWS];

    // Is the level-l block of nr x nc values at (i, j) stored?  (Tiles keep
    // less halo than they load below the levels analysed in LDS.)
    template <int l>
    static __device__ __forceinline__ bool stored(int i, int j, int nr, int nc) {
        if constexpr (!HALO || (A0 >> l) == G::sh(l)) {
            return true;
        } else {
            constexpr int a = G::sh(l);
            return i >= -a && i + nr <= G::hl(l) + a && j >= -a && j + nc <= G::wl(l) + a;
        }
    }

    // Whole planes: the loads of planes b0..b0+P-1 through a buffer
    // resource, with no branch (items past ITEMS and planes past B read
    // zeros).  RAG: planes stored as Hs x Ws corners (Rag), read one element
    // at a time, zero past the corner.
    template <bool RAG = false>
    __device__ __forceinline__ void issue_buf(const T* __restrict__ src, int b0, int B, int C,
                                              int c, int tid, Rag rg = Rag{G::H, G::W}) {
        static_assert(G::HT == 0, "whole planes only");
        if constexpr (RAG) {
            issue_rag(src, b0, B, C, c, tid, rg);
            return;
        }
        const GroupSpan<G, T> g(src, b0, B, C, c);
        const rsrc_t rs = make_rsrc(g.base, g.bytes);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int item = tid + it * G::NT;
            const int cv = item % NV;
            const int rb = (item / NV) % RB;
            const int pl = item / (NV * RB);
            const bool in = ITEMS % G::NT == 0 || item < ITEMS;
            const int off = in ? ((pl * C * G::H + ROWS * rb) * G::W + cv * V) * int(sizeof(T))
                               : kOutOfRange;
#pragma unroll
            for (int k = 0; k < ROWS; ++k)
                r[it][k] = buf_load<V * int(sizeof(T))>(rs, off + (in ? k * G::W * int(sizeof(T)) : 0));
        }
    }

    __device__ __forceinline__ void issue_rag(const T* __restrict__ src, int b0, int B, int C,
                                              int c, int tid, Rag rg) {
        const GroupSpan<G, T> g(src, b0, B, C, c, rg.Hs * rg.Ws);
        const rsrc_t rs = make_rsrc(g.base, g.bytes);
        constexpr int ES = int(sizeof(T));
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int item = tid + it * G::NT;
            const int cv = item % NV;
            const int rb = (item / NV) % RB;
            const int pl = item / (NV * RB);
            const bool in = ITEMS % G::NT == 0 || item < ITEMS;
#pragma unroll
            for (int k = 0; k < ROWS; ++k) {
                const int rr = ROWS * rb + k;
                union {
                    raw_t raw;
                    T e[V];
                } u;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const int col = cv * V + e;
                    const bool ok = in && rr < rg.Hs && col < rg.Ws;
                    const int off = ok ? ((pl * C * rg.Hs + rr) * rg.Ws + col) * ES : kOutOfRange;
                    u.e[e] = buf_load_elem<T>(rs, off);
                }
                r[it][k] = u.raw;
            }
        }
    }

    // Tiles: the footprint of the tile at (y0, x0) of plane b through a
    // buffer resource over that plane; items outside the plane (and b >= B)
    // read zeros without a branch.  Hp, Wp, y0, x0 are multiples of 4 and of
    // V, so an item is entirely inside or entirely outside.
    __device__ __forceinline__ void issue_tile_buf(const T* __restrict__ src, int b, int B, int C,
                                                   int c, int tid, int y0, int x0, int Hp,
                                                   int Wp) {
        const T* base = src + (size_t(min(b, B - 1)) * C + c) * Hp * Wp;
        const rsrc_t rs = make_rsrc(base, b < B ? Hp * Wp * int(sizeof(T)) : 0);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int item = tid + it * G::NT;
            const int cv = item % NV;
            const int rb = (item / NV) % RB;
            const int yy = y0 - A0 + ROWS * rb, xx = x0 - A0 + cv * V;
            const bool in = (ITEMS % G::NT == 0 || item < ITEMS) && yy >= 0 && yy < Hp &&
                            xx >= 0 && xx < Wp;
            const int off = in ? (yy * Wp + xx) * int(sizeof(T)) : kOutOfRange;
#pragma unroll
            for (int k = 0; k < ROWS; ++k)
                r[it][k] = buf_load<V * int(sizeof(T))>(rs, off + (in ? k * Wp * int(sizeof(T)) : 0));
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

    // N consecutive coefficients of each subband of level l at row i,
    // columns j..j+N-1: to the x side (aligned rows) or the compact dy side.
    template <bool VSIDE, int l, int N>
    static __device__ __forceinline__ void put_row(float* lds, int pl, int i, int j,
                                                   const float (&sub)[4][N]) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if constexpr (VSIDE) {
                float* dst = lds + G::vidx(l, pl, sb, i, j);
#pragma unroll
                for (int m = 0; m < N; ++m) dst[m] = sub[sb][m];
            } else {
                lds_put<N, G::al(l)>(lds + G::uidx(l, pl, sb, i, j), sub[sb]);
            }
        }
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
                const int fy = ROWS * rb - A0, fx = cv * V - A0;
                if constexpr (WRITE_X) {
                    if (stored<0>(fy, fx, ROWS, V)) {
                        float* o = lds + G::uidx(0, pl, 0, fy, fx);
#pragma unroll
                        for (int k = 0; k < ROWS; ++k)
                            lds_put<V, G::al(0)>(o + k * G::pitch(0), x[k]);
                    }
                }
                if constexpr (G::L >= 1) {  // (L = 0: plain depthwise conv)
                    float ll[ROWS / 2][V / 2];
#pragma unroll
                    for (int rr = 0; rr < ROWS / 2; ++rr) {
                        float sub[4][V / 2];
#pragma unroll
                        for (int m = 0; m < V / 2; ++m) {
                            float o[4];
                            butterfly(x[2 * rr][2 * m], x[2 * rr][2 * m + 1], x[2 * rr + 1][2 * m],
                                      x[2 * rr + 1][2 * m + 1], o);
                            ll[rr][m] = o[0];
#pragma unroll
                            for (int sb = 0; sb < 4; ++sb) sub[sb][m] = o[sb];
                        }
                        if (VSIDE || stored<1>(fy / 2, fx / 2, ROWS / 2, V / 2))
                            put_row<VSIDE, 1, V / 2>(lds, pl, fy / 2 + rr, fx / 2, sub);
                    }
                    if constexpr (ROWS == 4) {
                        float sub[4][V / 4];
#pragma unroll
                        for (int m = 0; m < V / 4; ++m) {
                            float o[4];
                            butterfly(ll[0][2 * m], ll[0][2 * m + 1], ll[1][2 * m], ll[1][2 * m + 1], o);
#pragma unroll
                            for (int sb = 0; sb < 4; ++sb) sub[sb][m] = o[sb];
                        }
                        if (VSIDE || stored<2>(fy / 4, fx / 4, 1, V / 4))
                            put_row<VSIDE, 2, V / 4>(lds, pl, fy / 4, fx / 4, sub);
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
    constexpr int a = VSIDE ? 0 : G::ah(l);  // the dy side needs the core only
    constexpr int h = G::hl(l) + 2 * a, w = G::wl(l) + 2 * a, ITEMS = G::P * h * w;
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int item = tid + it * G::NT;
        if (ITEMS % G::NT == 0 || item < ITEMS) {
            const int j = item % w - a;
            const int i = (item / w) % h - a;
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
            const float a0 = s[0], b = s[1], c = s[sp], d = s[sp + 1];
            const float s0 = a0 + b, d0 = a0 - b, s1 = c + d, d1 = c - d;
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

// Sum of a lane's tile of values: each row in order, then the row sums
// pairwise.  A running total over many tiles then takes one addition per
// tile instead of one per value, which keeps its rounding error that of a
// run as long as the number of tiles.
template <int Q, int R>
__device__ __forceinline__ float tile_sum(const float (&d)[Q][R]) {
    float rs[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        float a = d[q][0];
#pragma unroll
        for (int j = 1; j < R; ++j) a += d[q][j];
        rs[q] = a;
    }
#pragma unroll
    for (int w = 1; w < Q; w *= 2)
#pragma unroll
        for (int q = 0; q + w < Q; q += 2 * w) rs[q] += rs[q + w];
    return rs[0];
}

// acc[q][j] = sum_{u,v} w[u*K+v] * src[(q+u)*pitch + j+v].  With CAPTURE the
// window's centre, the tile's own input values, is kept in ctr[q][j].
template <int K, int Q, int R, bool CAPTURE = false>
__device__ __forceinline__ void conv_tile(const float* src, int pitch, const float (&w)[K * K],
                                          float init, float (&acc)[Q][R],
                                          float (*ctr)[R] = nullptr) {
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
        if constexpr (CAPTURE) {
            constexpr int p = K / 2;
            if (ir >= p && ir < p + Q)
#pragma unroll
                for (int j = 0; j < R; ++j) ctr[ir - p][j] = in[j + p];
        }
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

// One pass over a tile's window serving two sums: the conv
// acc[q][j] = sum_{u,v} w[u*K+v] * src[(q+u)*pitch + j+v] and the
// correlation g[u*K+v] += sum_{q,j} a[q][j] * src[(q+u)*pitch + j+v]; ctr
// gets the window's centre (the tile's own input values).  The window is read
// one row ahead of the FMAs that use it and no further: after a row, an empty
// asm on every sum the row touched and on the next row's offset keeps the
// scheduler from hoisting later rows above it (volatile asm statements keep
// their order), so two rows are live instead of the whole window beside the
// 2 x (tile + taps) accumulators.
template <int K, int Q, int R>
__device__ __forceinline__ void conv_corr_tile(const float* src, int pitch,
                                               const float (&w)[K * K], const float (&a)[Q][R],
                                               float (&acc)[Q][R], float (&g)[K * K],
                                               float (&ctr)[Q][R]) {
    constexpr int p = K / 2, NR = Q + K - 1, NC = R + K - 1;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[q][j] = 0.f;
    float in[2][NC];
#pragma unroll
    for (int m = 0; m < NC; ++m) in[0][m] = src[m];
    int nxt = pitch;  // element offset of the next row
#pragma unroll
    for (int ir = 0; ir < NR; ++ir) {
        const float* cur = in[ir & 1];
        if (ir + 1 < NR) {
#pragma unroll
            for (int m = 0; m < NC; ++m) in[(ir + 1) & 1][m] = src[nxt + m];
            nxt += pitch;
        }
        if (ir >= p && ir < p + Q)
#pragma unroll
            for (int j = 0; j < R; ++j) ctr[ir - p][j] = cur[j + p];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        acc[q][j] = fmaf(w[u * K + v], cur[j + v], acc[q][j]);
                        g[u * K + v] = fmaf(a[q][j], cur[j + v], g[u * K + v]);
                    }
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int j = 0; j < R; ++j) asm volatile("" : "+v"(acc[q][j]));
#pragma unroll
                for (int v = 0; v < K; ++v) asm volatile("" : "+v"(g[u * K + v]));
            }
        }
        asm volatile("" : "+v"(nxt));
    }
}

// conv_corr_tile with the window's centre summed on the way (rows below
// nrows, columns below ncols) instead of kept: one register for the Q x R
// of the centre.
template <int K, int Q, int R>
__device__ __forceinline__ void conv_corr_tile_csum(const float* src, int pitch,
                                               const float (&w)[K * K], const float (&a)[Q][R],
                                               float (&acc)[Q][R], float (&g)[K * K],
                                               float& csum, int nrows, int ncols) {
    constexpr int p = K / 2, NR = Q + K - 1, NC = R + K - 1;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[q][j] = 0.f;
    float in[2][NC];
#pragma unroll
    for (int m = 0; m < NC; ++m) in[0][m] = src[m];
    int nxt = pitch;  // element offset of the next row
#pragma unroll
    for (int ir = 0; ir < NR; ++ir) {
        const float* cur = in[ir & 1];
        if (ir + 1 < NR) {
#pragma unroll
            for (int m = 0; m < NC; ++m) in[(ir + 1) & 1][m] = src[nxt + m];
            nxt += pitch;
        }
        if (ir >= p && ir < p + Q) {
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < R; ++j) rs += (ir - p < nrows && j < ncols) ? cur[j + p] : 0.f;
            csum += rs;
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        acc[q][j] = fmaf(w[u * K + v], cur[j + v], acc[q][j]);
                        g[u * K + v] = fmaf(a[q][j], cur[j + v], g[u * K + v]);
                    }
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int j = 0; j < R; ++j) asm volatile("" : "+v"(acc[q][j]));
#pragma unroll
                for (int v = 0; v < K; ++v) asm volatile("" : "+v"(g[u * K + v]));
            }
        }
        asm volatile("" : "+v"(nxt));
    }
}

// The correlation of conv_corr_tile alone (no conv): g[u*K+v] +=
// sum_{q,j} a[q][j] * src[(q+u)*pitch + j+v], ctr the window's centre, with
// the same one-row-ahead reads and fences.
template <int K, int Q, int R>
__device__ __forceinline__ void corr_window_tile(const float* src, int pitch,
                                                 const float (&a)[Q][R], float (&g)[K * K],
                                                 float (&ctr)[Q][R]) {
    constexpr int p = K / 2, NR = Q + K - 1, NC = R + K - 1;
    float in[2][NC];
#pragma unroll
    for (int m = 0; m < NC; ++m) in[0][m] = src[m];
    int nxt = pitch;
#pragma unroll
    for (int ir = 0; ir < NR; ++ir) {
        const float* cur = in[ir & 1];
        if (ir + 1 < NR) {
#pragma unroll
            for (int m = 0; m < NC; ++m) in[(ir + 1) & 1][m] = src[nxt + m];
            nxt += pitch;
        }
        if (ir >= p && ir < p + Q)
#pragma unroll
            for (int j = 0; j < R; ++j) ctr[ir - p][j] = cur[j + p];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K) {
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int j = 0; j < R; ++j)
                        g[u * K + v] = fmaf(a[q][j], cur[j + v], g[u * K + v]);
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = ir - q;
            if (u >= 0 && u < K)
#pragma unroll
                for (int v = 0; v < K; ++v) asm volatile("" : "+v"(g[u * K + v]));
        }
        asm volatile("" : "+v"(nxt));
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

// Output rows 2i and 2i+1, columns col .. col+CW-1 (of plane pl's core):
// the base conv in the level-0 array plus the synthesis of the convolved
// subbands (level 2, whose coarser levels are already folded into its LL,
// folded into the level-1 LL on the fly, then each level-1 coefficient
// expanded over its 2x2 block).
template <class G, int CW>
__device__ __forceinline__ void synth_rows(const float* lds, int pl, int i, int col,
                                           float (&r0)[CW], float (&r1)[CW]) {
    const float* x0 = lds + G::uidx(0, pl, 0, 2 * i, col);
    lds_get<CW, G::al(0)>(x0, r0);
    lds_get<CW, G::al(0)>(x0 + G::pitch(0), r1);
    if constexpr (G::L >= 1) {
        float cf[4][CW / 2];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
            lds_get<CW / 2, G::al(1)>(lds + G::uidx(1, pl, sb, i, col / 2), cf[sb]);
#pragma unroll
        for (int m = 0; m < CW / 2; ++m) {
            float ll = cf[0][m];
            if constexpr (G::L >= 2) {
                constexpr int A2 = G::arr(2);
                const int j = col / 2 + m;
                const float* c2 = lds + G::uidx(2, pl, 0, i >> 1, j >> 1);
                const float sy2 = (i & 1) ? -1.f : 1.f, sx2 = (j & 1) ? -1.f : 1.f;
                const float e2 = fmaf(sy2, c2[2 * A2], c2[0]);
                const float f2 = fmaf(sy2, c2[3 * A2], c2[A2]);
                ll += fmaf(sx2, f2, e2);
            }
            const float lh = cf[1][m], hl = cf[2][m], hh = cf[3][m];
            const float e0 = ll + hl, f0 = lh + hh;  // row 2i   (row bit 0)
            const float e1 = ll - hl, f1 = lh - hh;  // row 2i+1 (row bit 1)
            r0[2 * m] += e0 + f0;
            r0[2 * m + 1] += e0 - f0;
            r1[2 * m] += e1 + f1;
            r1[2 * m + 1] += e1 - f1;
        }
    }
}

// The synthesis and the store in one pass, through a buffer resource (no LDS
// write-back, no branch: lanes past ITEMS re-read a valid item and store out
// of range).  Whole planes (HT == 0): the group's planes.  Tiles: the core of
// the tile at (y0, x0) of plane b of an Hp x Wp tensor; rows and columns
// past the plane, and b >= B, store out of range.
template <class G, typename T, bool WIDE = false>
__device__ __forceinline__ void final_store(const float* lds, T* __restrict__ out, int b0, int B,
                                            int C, int c, int tid, int y0 = 0, int x0 = 0,
                                            int Hp = G::H, int Wp = G::W) {
    constexpr int V = vec_elems<T>(G::W);
    constexpr int NV = G::W / V, RP = G::H / 2, ITEMS = G::P * RP * NV;
    // columns per pass: at most 4 floats, so that an 8-wide fp16 item keeps
    // few values live (two 8-byte stores per row instead of one 16-byte);
    // WIDE: the whole item per pass, for kernels with registers to spare
    constexpr int CW = V < 4 || WIDE ? V : 4, NCH = V / CW;
    constexpr int BYTES = CW * int(sizeof(T));
    using raw_t = typename RawVec<BYTES>::type;
    rsrc_t rs;
    int row_elems;  // elements between two output rows
    if constexpr (G::HT == 0) {
        const GroupSpan<G, T> g(out, b0, B, C, c);
        rs = make_rsrc(g.base, g.bytes);
        row_elems = G::W;
    } else {
        const T* base = out + (size_t(min(b0, B - 1)) * C + c) * Hp * Wp;
        rs = make_rsrc(base, b0 < B ? Hp * Wp * int(sizeof(T)) : 0);
        row_elems = Wp;
    }
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int raw_item = tid + it * G::NT;
        bool in = ITEMS % G::NT == 0 || raw_item < ITEMS;
        const int item = in ? raw_item : ITEMS - 1;
        const int cv = item % NV;
        const int i = (item / NV) % RP;
        const int pl = item / (NV * RP);
        int off;
        if constexpr (G::HT == 0) {
            off = ((pl * C * G::H + 2 * i) * G::W + cv * V) * int(sizeof(T));
        } else {
            const int yy = y0 + 2 * i, xx = x0 + cv * V;
            in = in && yy < Hp && xx < Wp;
            off = (yy * Wp + xx) * int(sizeof(T));
        }
        off = in ? off : kOutOfRange;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            float r0[CW], r1[CW];
            synth_rows<G, CW>(lds, pl, i, cv * V + ch * CW, r0, r1);
            union {
                raw_t raw;
                T e[CW];
            } u0, u1;
            store_vec<T, CW>(u0.e, r0);
            store_vec<T, CW>(u1.e, r1);
            const int o = off + (in ? ch * BYTES : 0);
            // fp32 rows and whole 16-byte fp16 pieces go out non-temporal:
            // the layer's output is not read again by it, and streaming it
            // past the caches took the stage-1 forward 43.1 -> 41.6 us, 14²
            // 18.6 -> 17.6 us, the fp16 forward (whole items) 82.4 -> 80.5
            // us; fp16's 8-byte pieces were slower so (82.0 -> 82.5 us)
            constexpr int kAux = sizeof(T) == 4 || BYTES == 16 ? 2 : 0;
            buf_store<kAux>(u0.raw, rs, o);
            buf_store<kAux>(u1.raw, rs, o + (in ? row_elems * int(sizeof(T)) : 0));
        }
    }
}

// final_store for whole planes stored as Hs x Ws corners (Rag): the same
// synthesis, then one element at a time, only inside the corner.
template <class G, typename T>
__device__ __forceinline__ void final_store_rag(const float* lds, T* __restrict__ out, int b0,
                                                int B, int C, int c, int tid, Rag rg) {
    static_assert(G::HT == 0, "whole planes only");
    constexpr int V = vec_elems<T>(G::W);
    constexpr int NV = G::W / V, RP = G::H / 2, ITEMS = G::P * RP * NV;
    constexpr int CW = V < 4 ? V : 4, NCH = V / CW;
    constexpr int ES = int(sizeof(T));
    const GroupSpan<G, T> g(out, b0, B, C, c, rg.Hs * rg.Ws);
    const rsrc_t rs = make_rsrc(g.base, g.bytes);
#pragma unroll
    for (int it = 0; it < cdiv(ITEMS, G::NT); ++it) {
        const int raw_item = tid + it * G::NT;
        const bool in = ITEMS % G::NT == 0 || raw_item < ITEMS;
        const int item = in ? raw_item : ITEMS - 1;
        const int cv = item % NV;
        const int i = (item / NV) % RP;
        const int pl = item / (NV * RP);
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            float r0[CW], r1[CW];
            synth_rows<G, CW>(lds, pl, i, cv * V + ch * CW, r0, r1);
#pragma unroll
            for (int e = 0; e < CW; ++e) {
                const int col = cv * V + ch * CW + e;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rr = 2 * i + h;
                    const bool ok = in && rr < rg.Hs && col < rg.Ws;
                    const int off = ok ? ((pl * C * rg.Hs + rr) * rg.Ws + col) * ES : kOutOfRange;
                    buf_store_elem<T>(from_f<T>(h ? r1[e] : r0[e]), rs, off);
                }
            }
        }
    }
}

// Folded filters into LDS: [0, KK) base, then (l, s) blocks, then the bias.
// bb is read in either form (its value unused when FLIP), so it must point
// at C readable elements then too: the callers pass wb.  Each lane reads
// its two values (a tap and its scale, or the bias and
// beta) unconditionally, from addresses chosen per lane, and computes after
// both are issued: with beta read as a branch-guarded scalar and the taps
// read in the lanes' branches, a fold waited on two memory round trips.
template <class G, typename T, bool FLIP>
__device__ __forceinline__ void fold_weights(float* wf, const T* __restrict__ wb,
                                             const T* __restrict__ bb, const T* __restrict__ sb,
                                             const T* __restrict__ ww, const T* __restrict__ sw,
                                             int C, int c, int tid) {
    constexpr int KK = G::KK;
    for (int i = tid; i < G::NWF; i += G::NT) {
        const bool base = i < KK, wav = !base && i < G::NWF - 1;
        const int jj = wav ? i - KK : 0, ls = jj / KK, t = jj - ls * KK;
        const int l = ls >> 2, s = ls & 3;
        const size_t gi = (size_t(l) * C + c) * 4 + s;
        const int tb = FLIP ? KK - 1 - i : i, tw = FLIP ? KK - 1 - t : t;
        // sb == NULL: no base scale (the plain depthwise conv)
        const T* a0 = base ? wb + size_t(c) * KK + tb : wav ? ww + gi * KK + tw : bb + c;
        const T* a1 = wav ? sw + gi : sb ? sb + c : a0;
        const float r0 = to_f(*a0), r1 = to_f(*a1);
        const float beta = sb ? r1 : 1.f;
        float v;
        if (base)
            v = beta * r0;
        else if (wav)
            v = r1 * ldexpf(1.f, -2 * (l + 1)) * r0;
        else
            v = FLIP ? 0.f : beta * r0;
        wf[i] = v;
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Wave priority from here on (s_setprio, 0..3).  A SIMD issues from its ready
// waves in priority order, oldest first among equals; with three workgroups
// of one kernel per compute unit, each in its own phase of the per-group
// chain, the order decides whether a workgroup's short latency-bound phases
// (commits, write-back, synthesis and stores between barriers) wait behind
// another workgroup's FMAs.  The fences keep the compiler from moving
// instructions across the change.
template <int N>
__device__ __forceinline__ void wave_prio() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(N);
    __builtin_amdgcn_sched_barrier(0);
}

// Wait until every vector-memory access of this wave has completed.  gfx9
// counts loads and stores in one counter that drains in issue order, so the
// wait for the next group's prefetched loads, placed after this group's
// stores, also waits for those stores' write acknowledgements.  Called just
// before the stores (the loads, issued a write-back and a synthesis earlier,
// have arrived), it leaves no load outstanding behind them, and the next
// commit does not wait at all.
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Phase priorities (commit and analysis, conv, write-back to store) of the
// kernels that gain from them, chosen among 12 settings per kernel (stage 1
// unless named, gated per-call times, one box):
// - whole-plane forward: 3, 1, 0 -- the stores lowest (fp32 48.1 -> 44.8
//   us, fp16 92 -> 86 us, 28^2 30.4 -> 29.4 us); with the stores above the
//   conv it ran 46-49 us;
// - one-side whole-plane backward: fp32 0, 1, 3 (93.0 -> 84.6 us), fp16 3, 0,
//   3 (168 -> 151.5 us) -- the store phase highest;
// - two-side whole-plane backward: 0, 1, 3 (28^2: 56.3 -> 53.9 us, 14^2
//   40.7 -> 40.0 us);
// - tile forward: 0, 1, 3 (512^2: 552 -> 520 us);
// - tile backward: x's commit 2, dy's commit 3, conv 0, store 3 (512^2:
//   960 -> 944 us); a conv above the other phases slowed it by up to 20%.
struct PrioPlaneApply { static constexpr int commit = 3, conv = 1, store = 0; };
template <typename T>
struct PrioPlaneBwd1 {
    static constexpr bool f32 = std::is_same<T, float>::value;
    static constexpr int commit = f32 ? 0 : 3, conv = f32 ? 1 : 0, store = 3;
};
struct PrioPlaneBwd { static constexpr int commit = 0, conv = 1, store = 3; };
struct PrioTileApply { static constexpr int commit = 0, conv = 1, store = 3; };
struct PrioTileBwd1 { static constexpr int commit_x = 2, commit_dy = 3, conv = 0, store = 3; };

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
// is loaded into registers while the current one is computed; the output is
// synthesised and stored in one pass.  Loads and stores go through buffer
// resources with no branch, so the only wait before a group's input is used
// is for that input.
// Register budget of the forward: the waves per SIMD the LDS footprint
// allows, at most 3.  Shapes that fit 128 VGPRs keep four waves anyway; the
// ones that do not (the 56 x 56 stage shape among them) would spill at four,
// and each spilled register is a scratch store per thread of every
// workgroup, HBM writes beside the output, for no speed (at 127 VGPRs and
// four waves the stage-1 forward ran no faster than at three: its time is
// the latency of its per-group phase chain, not a lack of waves).
template <int K, int L, int H, int W, int P, int NT, typename T>
constexpr int apply_waves() {
    const int w = waves_for_lds(apply_lds_bytes<Geo<K, L, H, W, P, NT>>(), NT);
    constexpr int cap = 3;
    return w < cap ? w : cap;
}

template <int K, int L, int H, int W, int P, int NT, typename T, bool FLIP, bool RAG = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(
    apply_waves<K, L, H, W, P, NT, T>(), 8))) void k_plane_apply(
    const T* __restrict__ in, const T* __restrict__ wb, const T* __restrict__ bb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    T* __restrict__ out, int B, int C, Rag rg) {
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
    if (q0 < q1) fx.template issue_buf<RAG>(in, (q0 % ngroups) * P, B, C, q0 / ngroups, tid, rg);
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

    // fp16: the filters are reloaded from LDS before each group's conv
    // instead of living in registers across groups, which takes the fp16
    // forward from 152 to 127 VGPRs (no spills in its ragged form, which
    // spilled 148 bytes per lane: 55 x 55 forward 102 -> 64.5 us; stage 1
    // fp16 85.6 -> 84.0 us).  fp32 keeps them: on small planes the reload is
    // per-group work for few FMAs (28 x 28: 29.6 -> 30.9 us).
    constexpr bool kReload = std::is_same<T, __half>::value;
    float w[KK];
    float init = 0.f;
    int cur = -1;
    // the first group's loads, so that no path into the loop carries loads
    // whose wait would fall behind stores (drain_vmem)
    drain_vmem();
    for (int q = q0; q < q1; ++q) {
        const int c = q / ngroups;
        const int b0 = (q % ngroups) * P;
        if (c != cur) {
            fold_weights<G, T, FLIP>(wf, wb, bb, sb, ww, sw, C, c, tid);
            __syncthreads();
            if constexpr (!kReload) {
#pragma unroll
                for (int t = 0; t < KK; ++t) w[t] = wf[wsrc + t];
            }
            init = job.lvl == 0 ? wf[G::NWF - 1] : 0.f;
            cur = c;
        }
        wave_prio<PrioPlaneApply::commit>();
        fx.template commit<true, false>(lds, tid);
        __syncthreads();
        static_for<F::LEVELS + 1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            __syncthreads();
        });
        float acc[Q][R];
        wave_prio<PrioPlaneApply::conv>();
        if (job.on) {
            if constexpr (kReload) {
#pragma unroll
                for (int t = 0; t < KK; ++t) w[t] = wf[wsrc + t];
            }
            conv_tile<K, Q, R>(lds + win, pitch, w, init, acc);
        }
        wave_prio<PrioPlaneApply::store>();
        // the next group's loads fly during write-back, synthesis and store
        if (q + 1 < q1) fx.template issue_buf<RAG>(in, ((q + 1) % ngroups) * P, B, C, (q + 1) / ngroups, tid, rg);
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
        // level 1 inside final_store
        static_for<0, L - 2>([&](auto lc) {
            cascade_level<G, L - decltype(lc)::value>(lds, tid);
            __syncthreads();
        });
        drain_vmem();
        if constexpr (RAG)
            final_store_rag<G, T>(lds, out, b0, B, C, c, tid, rg);
        else
            final_store<G, T, std::is_same<T, __half>::value>(lds, out, b0, B, C, c, tid);
        __syncthreads();
    }
}

// Sum over a team of 8 consecutive lanes (aligned within a 16-lane DPP row),
// in a fixed order: two quad-permute steps leave every lane of a quad its
// quad's sum, then row_shr:4 hands lanes 4..7 of the team the first quad's,
// so lane 4 of the team holds the total (the other lanes hold partials).
__device__ __forceinline__ float team8_sum(float s) {
    constexpr int kXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
    constexpr int kXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
    constexpr int kShr4 = 0x114;  // row_shr:4
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), kXor1, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), kXor2, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), kShr4, 0xF, 0xF, false));
    return s;
}

// Fixed-order workgroup reduction of the lanes' tap accumulators into one
// partial row [G_b (KK), sum dy, G[l][s] (4 L KK)], zero-padded to npart
// floats.  The lanes stage their accumulators in LDS; then each entry is
// summed by a team of 8 lanes -- lane m of the team takes the entry's lanes
// m, m + 8, ... of its (array, subband) in order, and the team's sums meet
// in a DPP tree (team8_sum) -- so no lane walks a long serial chain and the
// order, hence every bit, is fixed.  Overwrites LDS from `lds` on; the
// caller has synchronised the workgroup.
template <class G>
__device__ __forceinline__ void reduce_row(float* lds, const float (&acc)[G::KK], float sdy,
                                           float* __restrict__ row, int npart, int tid) {
    constexpr int KK = G::KK, RS = KK + 1, TEAM = 8, TEAMS = G::NT / TEAM;
    static_assert(G::NT % TEAM == 0, "whole teams");
    float* red = lds;  // [NT][KK + 1]
#pragma unroll
    for (int t = 0; t < KK; ++t) red[tid * RS + t] = acc[t];
    red[tid * RS + KK] = sdy;
    __syncthreads();
    const int m = tid % TEAM;
    // a trip count uniform over the workgroup: every lane reaches the DPP
    // steps of every round
    for (int o0 = 0; o0 < npart; o0 += TEAMS) {
        const int o = o0 + tid / TEAM;
        float s = 0.f;
        if (o <= KK) {
            for (int t = G::jstart(0) + m; t < G::jstart(1); t += TEAM) s += red[t * RS + o];
        } else if (o < G::NPART) {
            const int r = o - KK - 1, ls = r / KK, tap = r % KK;
            const int l = (ls >> 2) + 1, sb = ls & 3;
            by_level<G>(l, [&](auto lc) {
                constexpr int lv = decltype(lc)::value;
                if constexpr (lv > 0) {
                    constexpr int per = G::NS(lv) * G::NG(lv);
                    for (int pl = 0; pl < G::P; ++pl) {
                        const int t0 = G::jstart(lv) + (pl * 4 + sb) * per;
                        for (int t = t0 + m; t < t0 + per; t += TEAM) s += red[t * RS + tap];
                    }
                }
                return 0;
            });
        }
        s = team8_sum(s);
        if (m == 4 && o < npart) row[o] = s;
    }
}

// Weight-gradient partial sums of channel blockIdx.x % C over the groups of
// chunk blockIdx.x / C: one row of G::NPART floats per workgroup,
// [G_b (KK), sum dy, G[l][s] (4 L KK)].
template <int K, int L, int H, int W, int P, int NT, typename T, bool RAG = false>
__global__ __launch_bounds__(NT) void k_plane_bww(
    const T* __restrict__ x,
                                                  const T* __restrict__ dy,
                                                  float* __restrict__ part, int B, int C,
                                                  int gpw, Rag rg) {
    using G = GeoGrad<K, L, H, W, P, NT>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    const int ngroups = cdiv(B, P);
    const int g0 = chunk * gpw;
    const int g1 = min(g0 + gpw, ngroups);
    Fetch<G, T> fx, fd;
    if (g0 < g1) {
        fx.template issue_buf<RAG>(x, g0 * P, B, C, c, tid, rg);
        fd.template issue_buf<RAG>(dy, g0 * P, B, C, c, tid, rg);
    }
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
            fx.template issue_buf<RAG>(x, b0 + P, B, C, c, tid, rg);
            fd.template issue_buf<RAG>(dy, b0 + P, B, C, c, tid, rg);
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
                // addresses are clamped into the tensor; padding, and with
                // RAG the part of the plane beyond the stored corner, reads as 0
                const int Hs = RAG ? rg.Hs : H, Ws = RAG ? rg.Ws : W;
                const int b = b0 + job.pl;
                const T* dp = dy + (size_t(min(b, B - 1)) * C + c) * Hs * Ws;
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        const int row = job.grp * Q + q, col = job.strip * R + j;
                        const bool ok = b < B && q < nrows && j < ncols && row < Hs && col < Ws;
                        const int yy = min(row, Hs - 1);
                        const int xx = min(col, Ws - 1);
                        const float v = to_f(dp[yy * Ws + xx]);
                        d[q][j] = ok ? v : 0.f;
                    }
                sdy += tile_sum<Q, R>(d);
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

    reduce_row<G>(lds, acc, sdy, part + (size_t(chunk) * C + c) * G::NPART, G::NPART, tid);
}

// Offset of the dy side of the fused backward's LDS: a second copy of the
// x-side layout, started on bank 0 so that both windows of a tile fall on
// the same banks.
template <class G>
constexpr int bwd_dy_base() { return cdiv(G::side, 32) * 32; }
template <class G>
constexpr size_t bwd_lds_bytes() {
    const size_t a = sizeof(float) * (bwd_dy_base<G>() + G::side + G::NWF);
    const size_t b = sizeof(float) * G::NT * (G::KK + 1);
    return a > b ? a : b;
}

// Rows of weight-gradient partials written by the fused backward.  The
// C * ceil(B/P) (channel, group) items, channel-major, are split into nwg
// equal contiguous ranges, one per workgroup; a workgroup writes one row for
// each channel its range touches, so channel c has rows from workgroups
// owner(c*ng) .. owner((c+1)*ng - 1), stored at row c * rmax + (w - first).
struct LinearRows {
    long total;  // items
    int nwg, ng, rmax;
    __host__ __device__ long q0(int w) const { return total * w / nwg; }
    // the workgroup whose range holds item q
    __host__ __device__ int owner(long q) const { return int(((q + 1) * nwg - 1) / total); }
    __host__ __device__ int first(int c) const { return owner(long(c) * ng); }
    __host__ __device__ int count(int c) const {
        return owner(long(c + 1) * ng - 1) - first(c) + 1;
    }
};

// Fused backward: input gradient and weight-gradient partials reading x and
// dy once.  Workgroup w takes the items [q0(w), q0(w+1)) of LinearRows.
// dy and x are analysed side by side in LDS; each lane reads the dy window
// of its tile for the rotated-filter conv of the input gradient, keeps the
// window's centre (its tile of dy, or of V^l_s) and correlates it with the x
// window of the same tile for the weight gradient.  The input gradient then
// goes through the same synthesis and store as the forward.  With
// CROSS, a range may span channels: entering a new channel, the finished
// channel's taps are reduced to its row and the filters are folded again;
// without, every range lies in one channel (nwg a multiple of C) and the
// loop carries none of that.
// Two workgroups per compute unit fit its LDS at the stage shapes: the
// register budget is held to that occupancy.
template <int K, int L, int H, int W, int P, int NT, typename T, bool CROSS, bool RAG = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void k_plane_bwd(
    const T* __restrict__ x, const T* __restrict__ dy, const T* __restrict__ wb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    T* __restrict__ dx, float* __restrict__ part, int B, int C, LinearRows rows, Rag rg) {
    using G = GeoGrad<K, L, H, W, P, NT>;
    using F = Fetch<G, T>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R, DY = bwd_dy_base<G>();
    extern __shared__ float lds[];
    // The dy side starts DY floats in: as a compile-time constant that
    // offset does not fit the 8-bit offsets of paired LDS reads and costs an
    // address add per pair; held in a register, each row needs one base.
    int dyo = DY;
    asm volatile("" : "+s"(dyo));
    float* ldy = lds + dyo;
    float* wf = lds + DY + G::side;
    const int tid = threadIdx.x;
    const int ngroups = cdiv(B, P);
    const long q0 = rows.q0(blockIdx.x);
    const int nitems = int(rows.q0(blockIdx.x + 1) - q0);
    // (channel, group) of the range's first item; later items step through
    // the groups without divisions
    int c = int(q0 / ngroups), grp = int(q0 % ngroups);
    F fx, fd;
    if (nitems > 0) {
        fx.template issue_buf<RAG>(x, grp * P, B, C, c, tid, rg);
        fd.template issue_buf<RAG>(dy, grp * P, B, C, c, tid, rg);
    }
    for (int i = tid; i < DY + G::side; i += NT) lds[i] = 0.f;

    const Job job = decode_job<G>(tid);
    const int wsrc = job.lvl == 0 ? 0 : KK * (1 + (job.lvl - 1) * 4 + job.s);
    const int win = window_index<G>(job);
    const int pitch = level_pitch<G>(job.lvl);
    const int hrows = by_level<G>(job.lvl, [](auto lc) { return G::hl(decltype(lc)::value); });
    const int wcols = by_level<G>(job.lvl, [](auto lc) { return G::wl(decltype(lc)::value); });
    const int nrows = min(Q, hrows - job.grp * Q);
    const int ncols = min(R, wcols - job.strip * R);
    const bool full = nrows == Q && ncols == R;
    const int dst = win + G::p * pitch + G::p;
    float gacc[KK];
    float sdy = 0.f;
    int cur = -1;
    if constexpr (!CROSS) {
        // one channel for the whole range: fold once, before the loop
        fold_weights<G, T, true>(wf, wb, wb, sb, ww, sw, C, c, tid);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < KK; ++t) gacc[t] = 0.f;
        cur = c;
    }

    // the first loads, so that no path into the loop carries loads whose
    // wait would fall behind stores (drain_vmem)
    drain_vmem();
    for (int it = 0; it < nitems; ++it) {
        const int b0 = grp * P;
        if (CROSS && c != cur) {
            if (cur >= 0) {
                // the finished channel's row; the arrays the reduction used
                // are zeroed again and the filters folded again below
                reduce_row<G>(lds, gacc, sdy,
                              part + (size_t(cur) * rows.rmax + (blockIdx.x - rows.first(cur))) *
                                         G::NPART,
                              G::NPART, tid);
                __syncthreads();
                constexpr int RED = NT * (KK + 1) < DY + G::side ? NT * (KK + 1) : DY + G::side;
                for (int i = tid; i < RED; i += NT) lds[i] = 0.f;
            }
            fold_weights<G, T, true>(wf, wb, wb, sb, ww, sw, C, c, tid);
            __syncthreads();
#pragma unroll
            for (int t = 0; t < KK; ++t) gacc[t] = 0.f;
            sdy = 0.f;
            cur = c;
        }
        wave_prio<PrioPlaneBwd::commit>();
        fx.template commit<true, false>(lds, tid);
        fd.template commit<true, false>(ldy, tid);
        __syncthreads();
        static_for<F::LEVELS + 1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            analysis_level<G, decltype(lc)::value, false>(ldy, tid);
            __syncthreads();
        });
        float acc[Q][R];
        wave_prio<PrioPlaneBwd::conv>();
        if (job.on) {
            // The tile's own dy values (V^l_s at level l), read from the
            // core of its array: outside a level's core the arrays hold
            // zeros, so a partial tile needs no mask.  The weight taps come
            // first and the rotated-filter conv second, with the filters read
            // from LDS just before it (the empty asm keeps those reads and
            // the dy window's after the correlation): neither the filters nor
            // the conv sums are live beside the correlation's accumulators.
            float d[Q][R];
#pragma unroll
            for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                for (int j = 0; j < R; ++j) d[qq][j] = ldy[dst + qq * pitch + j];
            if (job.lvl == 0) sdy += tile_sum<Q, R>(d);
            corr_tile<K, Q, R>(d, lds + win, pitch, gacc);
            int wo = wsrc, yw = win;
            asm volatile("" : "+v"(wo));
            asm volatile("" : "+v"(yw));
            float w[KK];
#pragma unroll
            for (int t = 0; t < KK; ++t) w[t] = wf[wo + t];
            conv_tile<K, Q, R>(ldy + yw, pitch, w, 0.f, acc);
        }
        wave_prio<PrioPlaneBwd::store>();
        const bool wrap = grp + 1 == ngroups;
        const int cn = wrap ? c + 1 : c, gn = wrap ? 0 : grp + 1;
        if (it + 1 < nitems) {
            fx.template issue_buf<RAG>(x, gn * P, B, C, cn, tid, rg);
            fd.template issue_buf<RAG>(dy, gn * P, B, C, cn, tid, rg);
        }
        __syncthreads();
        if (job.on) {
            if (full) {
#pragma unroll
                for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                    for (int j = 0; j < R; ++j) ldy[dst + qq * pitch + j] = acc[qq][j];
            } else {
#pragma unroll
                for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                    for (int j = 0; j < R; ++j)
                        if (qq < nrows && j < ncols) ldy[dst + qq * pitch + j] = acc[qq][j];
            }
        }
        __syncthreads();
        static_for<0, L - 2>([&](auto lc) {
            cascade_level<G, L - decltype(lc)::value>(ldy, tid);
            __syncthreads();
        });
        drain_vmem();
        if constexpr (RAG)
            final_store_rag<G, T>(ldy, dx, b0, B, C, c, tid, rg);
        else
            final_store<G, T>(ldy, dx, b0, B, C, c, tid);
        c = cn;
        grp = gn;
        __syncthreads();
    }
    if (cur >= 0)
        reduce_row<G>(lds, gacc, sdy,
                      part + (size_t(cur) * rows.rmax + (blockIdx.x - rows.first(cur))) * G::NPART,
                      G::NPART, tid);
}

// LDS of the one-side fused backward: one array layout that x passes through
// before dy, the folded filters after it; the reduction rows reuse the start.
template <class G>
constexpr size_t bwd1_lds_bytes() {
    const size_t a = sizeof(float) * (G::side + G::NWF);
    const size_t b = sizeof(float) * G::NT * (G::KK + 1);
    return a > b ? a : b;
}

// Waves per SIMD for its register budget: what the LDS allows, at most 3.
template <class G>
constexpr int bwd1_waves() {
    const int w = waves_for_lds(bwd1_lds_bytes<G>(), G::NT);
    return w < 3 ? w : 3;
}

// Fused backward with one LDS side.  The weight taps are taken transposed:
// dK[u][v] = sum_{m,n} U[m][n] V[m-u+p][n-v+p] (U: x's subband, V: dy's), so
// a lane needs x only at its own tile (U[q][j], read from the arrays after x
// is analysed into them) and reads one window, of dy, for both the
// rotated-filter conv of the input gradient and the taps: tap (u, v) meets
// the window at row q + K-1-u, column j + K-1-v, so the taps accumulate in
// rotated order (gacc[KK-1-t] is tap t) with the conv's access pattern.  x
// goes through the arrays, then dy: half the LDS of two sides, which lets
// three workgroups share a compute unit, and half the window reads.  Items
// and CROSS as in k_plane_bwd; the register budget is held to the waves per
// SIMD the LDS allows, at most three.  Without DX the kernel is the weight
// gradient alone (wtconv_bwd_weight): no conv, no input gradient, `dx` and
// the filters unread.
template <int K, int L, int H, int W, int P, int NT, typename T, bool CROSS, bool DX = true,
          bool RAG = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(
    bwd1_waves<Geo<K, L, H, W, P, NT>>()))) void k_plane_bwd1(
    const T* __restrict__ x, const T* __restrict__ dy, const T* __restrict__ wb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    T* __restrict__ dx, float* __restrict__ part, int B, int C, LinearRows rows, Rag rg) {
    using G = Geo<K, L, H, W, P, NT>;
    using F = Fetch<G, T>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    float* wf = lds + G::side;
    const int tid = threadIdx.x;
    const int ngroups = cdiv(B, P);
    const long q0 = rows.q0(blockIdx.x);
    const int nitems = int(rows.q0(blockIdx.x + 1) - q0);
    int c = int(q0 / ngroups), grp = int(q0 % ngroups);
    F fx, fd;
    if (nitems > 0) {
        fx.template issue_buf<RAG>(x, grp * P, B, C, c, tid, rg);
        fd.template issue_buf<RAG>(dy, grp * P, B, C, c, tid, rg);
    }
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
    const int dst = win + G::p * pitch + G::p;
    float gacc[KK];  // rotated: gacc[KK - 1 - t] accumulates tap t
    float sdy = 0.f;
    int cur = -1;
    // the finished channel's partial row, taps back in order
    auto flush = [&](int ch) {
        float g[KK];
#pragma unroll
        for (int t = 0; t < KK; ++t) g[t] = gacc[KK - 1 - t];
        reduce_row<G>(lds, g, sdy,
                      part + (size_t(ch) * rows.rmax + (blockIdx.x - rows.first(ch))) * G::NPART,
                      G::NPART, tid);
    };
    if constexpr (!CROSS) {
        if constexpr (DX) fold_weights<G, T, true>(wf, wb, wb, sb, ww, sw, C, c, tid);
        // also orders the zeroing above before the first commit
        __syncthreads();
#pragma unroll
        for (int t = 0; t < KK; ++t) gacc[t] = 0.f;
        cur = c;
    }

    // the first group's loads, so that no path into the loop carries loads
    // whose wait would fall behind stores (drain_vmem)
    drain_vmem();
    for (int it = 0; it < nitems; ++it) {
        const int b0 = grp * P;
        int t = tid;
        if (CROSS && c != cur) {
            if (cur >= 0) {
                // the reduction overwrites the head of the arrays: zeroed
                // again (their borders must read zeros), filters folded again
                flush(cur);
                __syncthreads();
                constexpr int RED = NT * (KK + 1) < G::side ? NT * (KK + 1) : G::side;
                for (int i = tid; i < RED; i += NT) lds[i] = 0.f;
            }
            if constexpr (DX) fold_weights<G, T, true>(wf, wb, wb, sb, ww, sw, C, c, tid);
            __syncthreads();
#pragma unroll
            for (int t = 0; t < KK; ++t) gacc[t] = 0.f;
            sdy = 0.f;
            cur = c;
        }
        // x through the arrays: the lane keeps U at its tile (zeros outside
        // the level's core, so a partial tile needs no mask)
        wave_prio<PrioPlaneBwd1<T>::commit>();
        fx.template commit<true, false>(lds, t);
        __syncthreads();
        static_for<F::LEVELS + 1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, t);
            __syncthreads();
        });
        float u[Q][R];
        if (job.on)
#pragma unroll
            for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                for (int j = 0; j < R; ++j) u[qq][j] = lds[dst + qq * pitch + j];
        __syncthreads();
        // then dy: one window for the input-gradient conv and the taps
        fd.template commit<true, false>(lds, t);
        __syncthreads();
        static_for<F::LEVELS + 1, L + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, t);
            __syncthreads();
        });
        float acc[Q][R];
        if (job.on) {
            float d[Q][R];
            if constexpr (DX) {
                float w[KK];
#pragma unroll
                for (int t = 0; t < KK; ++t) w[t] = wf[wsrc + t];
                wave_prio<PrioPlaneBwd1<T>::conv>();
                conv_corr_tile<K, Q, R>(lds + win, pitch, w, u, acc, gacc, d);
                wave_prio<PrioPlaneBwd1<T>::store>();
            } else {
                corr_window_tile<K, Q, R>(lds + win, pitch, u, gacc, d);
            }
            if (job.lvl == 0) sdy += tile_sum<Q, R>(d);
        }
        const bool wrap = grp + 1 == ngroups;
        const int cn = wrap ? c + 1 : c, gn = wrap ? 0 : grp + 1;
        // The next group's loads, after the FMAs (the offset fence follows
        // the accumulator fences of the tile pass) and unconditional: past
        // the range's last item they cover no planes (b0 = B: an empty
        // buffer range, every load reads zero without touching memory).
        // Skipped loads would keep this group's registers live, around the
        // loop, beside the accumulators.
        asm volatile("" : "+v"(t));
        {
            const bool more = it + 1 < nitems;
            fx.template issue_buf<RAG>(x, more ? gn * P : B, B, C, more ? cn : c, t, rg);
            fd.template issue_buf<RAG>(dy, more ? gn * P : B, B, C, more ? cn : c, t, rg);
        }
        __syncthreads();
        if constexpr (DX) {
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
            static_for<0, L - 2>([&](auto lc) {
                cascade_level<G, L - decltype(lc)::value>(lds, t);
                __syncthreads();
            });
            drain_vmem();
            if constexpr (RAG)
                final_store_rag<G, T>(lds, dx, b0, B, C, c, t, rg);
            else
                final_store<G, T>(lds, dx, b0, B, C, c, t);
            __syncthreads();
        }
        c = cn;
        grp = gn;
    }
    if (cur >= 0) flush(cur);
}

// Sum the partial rows of each channel in order and apply the chain rule
// through the fold: dKb = beta G_b, dbias = beta sum dy,
// dbeta = <Kb, G_b> + bias sum dy, dK[l,s] = gamma 4^-l G[l,s],
// dgamma[l,s] = 4^-l <K[l,s], G[l,s]>.  Rows of channel c: with
// rows.nwg = 0, `nchunk` rows at (chunk * C + c); otherwise the LinearRows
// rows of c.  nchunk = 0 (and rows.nwg = 0) gives zero gradients.  The row
// sums and the products are taken in fp64 and rounded once to the output
// type.
// The workgroup is a chain of memory round trips, so it is laid out to
// have few: every device-memory read (rows, filters, scales, beta, bias) is
// issued by the lanes in one pass before the one barrier (beta and the bias
// by two lanes with the scales: read as branch-guarded scalars each was a
// round trip of its own ahead of the rows), and after it each thread
// computes one output and stores it once, last (stores count in vmcnt: a
// thread that stored and then went on to another output waited at its next
// vmcnt wait for the store's write acknowledgement, one round trip per
// output group).  The kernel size is a template argument so that the dot
// products unroll.  Up to kFinalNT threads: one per column of the rows and
// one per output (547 outputs at 512², L = 5, k = 5, in one pass).
constexpr int kFinalNT = 1024, kFinalRows = 16;

// Threads of k_bww_final for kernel size k and L levels: one per row column
// and one per output, in whole wavefronts.
__host__ __device__ constexpr int bww_final_threads(int k, int L) {
    const int KK = k * k, n = KK + 2 + 4 * L * KK + 4 * L;  // >= the row columns
    return n < kFinalNT ? (n + 63) / 64 * 64 : kFinalNT;
}

template <typename T, int K>
__global__ __launch_bounds__(kFinalNT) void k_bww_final(
    const float* __restrict__ part, int nchunk, LinearRows rows, int C, int L,
    const T* __restrict__ wb, const T* __restrict__ bb, const T* __restrict__ sb,
    const T* __restrict__ ww, const T* __restrict__ sw, T* __restrict__ dwb,
    T* __restrict__ dbb, T* __restrict__ dsb, T* __restrict__ dww, T* __restrict__ dsw) {
    // [NPART] row sums (fp64), then the filters Kb [KK], K [4 L KK], the
    // scales gamma [4 L], beta and the bias (fp32)
    extern __shared__ double gsum[];
    constexpr int KK = K * K;
    const int NPART = KK + 1 + 4 * L * KK, NF = KK + 4 * L * KK, NS = 4 * L;
    const int c = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    float* kf = reinterpret_cast<float*>(gsum + NPART);
    float* gam = kf + NF;
    const bool lin = rows.nwg > 0;
    const int nrow = lin ? rows.count(c) : nchunk;
    const size_t base = lin ? size_t(c) * rows.rmax : size_t(c);
    const size_t step = lin ? 1 : size_t(C);
    const int nmax = NF > NPART ? NF : NPART;  // >= NS + 2
    for (int i = tid; i < nmax; i += nt) {
        // every read below is unconditional, from an address chosen per lane
        // (a valid stand-in where the lane has no value), and selected after:
        // reads in the arms of branches were each waited for at the join,
        // one round trip apiece, before the rows were even issued
        const int fi = i < NF ? i : NF - 1;
        const int j = fi < KK ? 0 : fi - KK, ls = j / KK, t = j - ls * KK;
        const T* fsrc = fi < KK ? wb + size_t(c) * KK + fi
                                : ww + ((size_t(ls >> 2) * C + c) * 4 + (ls & 3)) * KK + t;
        // scales gamma, then beta (sb == NULL: no base scale, the plain
        // depthwise conv, and no dsb) and the bias
        const T* ssrc = i < NS                 ? sw + (size_t(i >> 2) * C + c) * 4 + (i & 3)
                        : (i == NS && sb)      ? sb + c
                        : (i == NS + 1 && dsb) ? bb + c
                                               : wb + size_t(c) * KK;
        const float f = to_f(*fsrc), sv = to_f(*ssrc);
        double acc = 0.0;
        if (i < NPART) {
            // kFinalRows rows per round, loaded unconditionally (a row index
            // past the last reads the last row again and is masked), so that
            // the round's loads are in flight together; added in row order
            for (int ch0 = 0; ch0 < nrow; ch0 += kFinalRows) {
                float v[kFinalRows];
#pragma unroll
                for (int u = 0; u < kFinalRows; ++u) {
                    const int r = min(ch0 + u, nrow - 1);
                    v[u] = part[(base + size_t(r) * step) * NPART + i];
                }
#pragma unroll
                for (int u = 0; u < kFinalRows; ++u) acc += ch0 + u < nrow ? double(v[u]) : 0.0;
            }
            gsum[i] = acc;
        }
        // (selected only now: the compiler makes the selects branches, and
        // a branch on a value waits for its read)
        const float sc = i < NS ? sv : i == NS ? (sb ? sv : 1.f) : (dsb ? sv : 0.f);
        if (i < NF) kf[i] = f;
        if (i < NS + 2) gam[i] = sc;
    }
    __syncthreads();
    const float beta = gam[NS], bias = gam[NS + 1];
    // outputs: dKb [KK], dbias, dbeta, dK [4 L KK], dgamma [4 L]
    const int nwv = 4 * L * KK, nout = KK + 2 + nwv + NS;
    for (int o = tid; o < nout; o += nt) {
        T* dst = nullptr;
        double v = 0.0;
        if (o < KK) {
            dst = dwb + size_t(c) * KK + o;
            v = beta * gsum[o];
        } else if (o == KK) {
            dst = dbb + c;
            v = beta * gsum[KK];
        } else if (o == KK + 1) {
            if (dsb) {
                double dot = double(bias) * gsum[KK];
#pragma unroll
                for (int t = 0; t < KK; ++t) dot += double(kf[t]) * gsum[t];
                dst = dsb + c;
                v = dot;
            }
        } else if (o < KK + 2 + nwv) {
            const int i = o - KK - 2, ls = i / KK, t = i % KK, l = ls >> 2, s = ls & 3;
            dst = dww + ((size_t(l) * C + c) * 4 + s) * KK + t;
            v = double(gam[ls]) * ldexp(1.0, -2 * (l + 1)) * gsum[KK + 1 + i];
        } else {
            const int i = o - KK - 2 - nwv, l = i >> 2, s = i & 3;
            double dot = 0.0;
#pragma unroll
            for (int t = 0; t < KK; ++t)
                dot += double(kf[KK + i * KK + t]) * gsum[KK + 1 + i * KK + t];
            dst = dsw + (size_t(l) * C + c) * 4 + s;
            v = ldexp(1.0, -2 * (l + 1)) * dot;
        }
        if (dst) *dst = from_f<T>(float(v));
    }
}

// ---------------------------------------------------------------------------
// Tiles of large planes
// ---------------------------------------------------------------------------

// Contribution of the levels deeper than the tile's (computed per plane by
// the deep kernels, fp32 at level-LT resolution) added to the level-LT LL
// coefficients of the tile's core.
// Position of a tile-kernel unit: channel, image, tile row and column, the
// column fastest.  Decoded from a unit index once per workgroup and then
// stepped, so the loop carries no divisions.
struct TileCursor {
    int c, b, ty, tx;
    __device__ static TileCursor at(long q, int B, int nty, int ntx) {
        const long per_c = long(B) * nty * ntx;
        const long r = q % per_c;
        const int t = int(r % (long(nty) * ntx));
        return TileCursor{int(q / per_c), int(r / (long(nty) * ntx)), t / ntx, t % ntx};
    }
    __device__ TileCursor next(int B, int nty, int ntx) const {
        TileCursor n = *this;
        if (++n.tx == ntx) {
            n.tx = 0;
            if (++n.ty == nty) {
                n.ty = 0;
                if (++n.b == B) {
                    n.b = 0;
                    ++n.c;
                }
            }
        }
        return n;
    }
};

// The deeper levels' contribution to a tile's level-LT LL core, in two
// halves: fetch_deep loads it into registers when a tile starts (so the load
// is in flight during the conv), add_deep adds it to LDS after the conv
// results are written.
template <class G>
struct DeepRegs {
    static constexpr int LT = G::L, h = G::hl(LT), w = G::wl(LT), ITEMS = h * w;
    static constexpr int N = cdiv(ITEMS, G::NT);
    float v[N];
};

template <class G>
__device__ __forceinline__ void fetch_deep(DeepRegs<G>& r, const float* __restrict__ deep, int b,
                                           int C, int c, int y0, int x0, int Hp, int Wp,
                                           int tid) {
    using D = DeepRegs<G>;
    constexpr int LT = D::LT;
    const int hd = Hp >> LT, wd = Wp >> LT;
    const float* dp = deep + (size_t(b) * C + c) * hd * wd;
#pragma unroll
    for (int n = 0; n < D::N; ++n) {
        const int item = tid + n * G::NT;
        const int i = item / D::w, j = item % D::w;
        const int gy = (y0 >> LT) + i, gx = (x0 >> LT) + j;
        r.v[n] = item < D::ITEMS && gy < hd && gx < wd ? dp[gy * wd + gx] : 0.f;
    }
}

template <class G>
__device__ __forceinline__ void add_deep(float* lds, const DeepRegs<G>& r, int tid) {
    using D = DeepRegs<G>;
#pragma unroll
    for (int n = 0; n < D::N; ++n) {
        const int item = tid + n * G::NT;
        if (item < D::ITEMS) lds[G::uidx(D::LT, 0, 0, item / D::w, item % D::w)] += r.v[n];
    }
}

// Forward (FLIP = false) or input gradient (FLIP = true) of the base conv and
// levels 1..LT on TH x TW output tiles of Hp x Wp planes; `deep` (may be null)
// holds levels LT+1..L.  (channel, image, tile) units, channel-major, are split
// into gridDim.x equal ranges.
template <int K, int LT, int TH, int TW, int NT, typename T, bool FLIP>
__global__ __launch_bounds__(NT) void k_tile_apply(
    const T* __restrict__ in, const T* __restrict__ wb, const T* __restrict__ bb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    const float* __restrict__ deep, T* __restrict__ out, int B, int C, int Hp, int Wp) {
    using G = GeoTileTrim<K, LT, TH, TW, NT>;
    using F = Fetch<G, T>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    float* wf = lds + G::side;
    const int tid = threadIdx.x;
    const int ntx = cdiv(Wp, TW), nty = cdiv(Hp, TH);
    const long per_c = long(B) * nty * ntx;
    const long total = long(C) * per_c;
    const long q0 = total * blockIdx.x / gridDim.x;
    const long q1 = total * (blockIdx.x + 1) / gridDim.x;
    TileCursor cu = TileCursor::at(q0, B, nty, ntx);
    F fx;
    if (q0 < q1) fx.issue_tile_buf(in, cu.b, B, C, cu.c, tid, cu.ty * TH, cu.tx * TW, Hp, Wp);
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
    const int dst = win + G::p * pitch + G::p;

    float w[KK];
    float init = 0.f;
    int cur = -1;
    // the first loads, so that no path into the loop carries loads whose
    // wait would fall behind stores (drain_vmem)
    drain_vmem();
    for (long q = q0; q < q1; ++q) {
        const int c = cu.c, b = cu.b, y0 = cu.ty * TH, x0 = cu.tx * TW;
        const TileCursor nx = cu.next(B, nty, ntx);
        if (c != cur) {
            fold_weights<G, T, FLIP>(wf, wb, bb, sb, ww, sw, C, c, tid);
            __syncthreads();
#pragma unroll
            for (int t = 0; t < KK; ++t) w[t] = wf[wsrc + t];
            init = job.lvl == 0 ? wf[G::NWF - 1] : 0.f;
            cur = c;
        }
        wave_prio<PrioTileApply::commit>();
        fx.template commit<true, false>(lds, tid);
        __syncthreads();
        static_for<F::LEVELS + 1, LT + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            __syncthreads();
        });
        DeepRegs<G> dr;
        if (deep) fetch_deep<G>(dr, deep, b, C, c, y0, x0, Hp, Wp, tid);
        float acc[Q][R];
        wave_prio<PrioTileApply::conv>();
        if (job.on) conv_tile<K, Q, R>(lds + win, pitch, w, init, acc);
        wave_prio<PrioTileApply::store>();
        // unconditional (past the range it covers an empty buffer range:
        // b = B), so that every path carries the same loads: with the load
        // on one path only, the wait for the deeper levels' value after it
        // could only be vmcnt(0), a wait for this prefetch as well
        const bool more = q + 1 < q1;
        fx.issue_tile_buf(in, more ? nx.b : B, B, C, nx.c, tid, nx.ty * TH, nx.tx * TW, Hp, Wp);
        __syncthreads();
        if (job.on) {
#pragma unroll
            for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                for (int j = 0; j < R; ++j)
                    if (full || (qq < nrows && j < ncols)) lds[dst + qq * pitch + j] = acc[qq][j];
        }
        __syncthreads();
        if (deep) {
            add_deep<G>(lds, dr, tid);
            __syncthreads();
        }
        static_for<0, LT - 2>([&](auto lc) {
            cascade_level<G, LT - decltype(lc)::value>(lds, tid);
            __syncthreads();
        });
        drain_vmem();
        final_store<G, T>(lds, out, b, B, C, c, tid, y0, x0, Hp, Wp);
        cu = nx;
        __syncthreads();
    }
}

// Weight-gradient partial sums of the base and levels 1..LT over the tiles of
// channel blockIdx.x % C: chunk blockIdx.x / C covers `upw` (image, tile)
// units.  One row of G::NPART floats per workgroup (levels past LT are left 0).
template <int K, int LT, int TH, int TW, int NT, typename T>
__global__ __launch_bounds__(NT) void k_tile_bww(const T* __restrict__ x,
                                                 const T* __restrict__ dy,
                                                 float* __restrict__ part, int B, int C, int Hp,
                                                 int Wp, int upw, int npart) {
    using G = Geo<K, LT, TH, TW, 1, NT, LT>;
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    const int ntx = cdiv(Wp, TW), nty = cdiv(Hp, TH);
    const int units = B * nty * ntx;
    const int u0 = chunk * upw;
    const int u1 = min(u0 + upw, units);
    TileCursor cu = TileCursor::at(u0, B, nty, ntx);  // c stays 0: one channel
    Fetch<G, T, true> fx;
    Fetch<G, T, false> fd;
    if (u0 < u1) {
        fx.issue_tile_buf(x, cu.b, B, C, c, tid, cu.ty * TH, cu.tx * TW, Hp, Wp);
        fd.issue_tile_buf(dy, cu.b, B, C, c, tid, cu.ty * TH, cu.tx * TW, Hp, Wp);
    }
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

    for (int u = u0; u < u1; ++u) {
        const int b = cu.b, y0 = cu.ty * TH, x0 = cu.tx * TW;
        const TileCursor nx = cu.next(B, nty, ntx);
        fx.template commit<true, false>(lds, tid);
        fd.template commit<false, true>(lds, tid);
        if (u + 1 < u1) {
            fx.issue_tile_buf(x, nx.b, B, C, c, tid, nx.ty * TH, nx.tx * TW, Hp, Wp);
            fd.issue_tile_buf(dy, nx.b, B, C, c, tid, nx.ty * TH, nx.tx * TW, Hp, Wp);
        }
        __syncthreads();
        static_for<Fetch<G, T, true>::LEVELS + 1, LT + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, tid);
            if constexpr (decltype(lc)::value > Fetch<G, T, false>::LEVELS)
                analysis_level<G, decltype(lc)::value, true>(lds, tid);
            __syncthreads();
        });
        static_for<Fetch<G, T, false>::LEVELS + 1, Fetch<G, T, true>::LEVELS + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, true>(lds, tid);
            __syncthreads();
        });
        if (job.on) {
            float d[Q][R];
            if (job.lvl == 0) {
                const T* dp = dy + (size_t(b) * C + c) * Hp * Wp;
#pragma unroll
                for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        const int yy = y0 + job.grp * Q + qq, xx = x0 + job.strip * R + j;
                        const bool ok = qq < nrows && j < ncols && yy < Hp && xx < Wp;
                        const float v = to_f(dp[min(yy, Hp - 1) * Wp + min(xx, Wp - 1)]);
                        d[qq][j] = ok ? v : 0.f;
                    }
                sdy += tile_sum<Q, R>(d);
            } else {
#pragma unroll
                for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                    for (int j = 0; j < R; ++j) d[qq][j] = lds[vsrc + qq * vp + j];
            }
            corr_tile<K, Q, R>(d, lds + win, pitch, acc);
        }
        cu = nx;
        __syncthreads();
    }

    reduce_row<G>(lds, acc, sdy, part + (size_t(chunk) * C + c) * npart, npart, tid);
}
}  // namespace dev
}  // namespace wtc

namespace wtc {
namespace dev {

// LDS of the one-side tile backward: one array layout (x's core, then dy with
// its halos) with the folded filters after it, or the reduction rows,
// whichever is larger.
template <class G>
constexpr size_t tile_bwd1_lds_bytes() {
    const size_t a = sizeof(float) * (G::side + G::NWF);
    const size_t b = sizeof(float) * G::NT * (G::KK + 1);
    return a > b ? a : b;
}
// Waves per SIMD for the register budget: what the LDS allows, at most 3,
// and 2 for 7 x 7 filters (their 49 taps and wider windows need the 256
// VGPRs of two waves; at three they spill).
template <class G>
constexpr int tile_bwd1_waves() {
    const int w = waves_for_lds(tile_bwd1_lds_bytes<G>(), G::NT);
    const int cap = G::K >= 7 ? 2 : 3;
    return w < cap ? w : cap;
}

// Fused backward of a large plane's tiles: the input gradient of the base
// conv and levels 1..LT (plus the deep levels' contribution `deep`, NULL if
// none) and the weight-gradient partials of those levels, reading x and dy
// once; with `px` (NULL: none) also the box sums U^LT_LL(x) of the planes.
// (channel, chunk) workgroups as in k_tile_bww.  One LDS side and transposed
// weight taps (as k_plane_bwd1): a lane needs x's subbands only at its own
// outputs, which lie in the tile's core, and the tile is aligned to 2^LT, so
// x is loaded and analysed for the core alone (a quarter of the footprint
// at 32 x 32, LT = 3) and each lane keeps U at its tile, masked to its part
// of the core; then dy, with the halos, goes through the same arrays and
// one window per tile feeds the input-gradient conv and the taps.  Levels
// beyond the fetch's are analysed over their halos for x too, from stale
// values there: only core coefficients, which depend on core values alone,
// are read.  Registers for up to three waves per SIMD where the LDS allows
// (the trimmed layout of the forward): at k = 5 that holds without spills
// because nothing long-lived shares the peaks -- the filters are reloaded
// from LDS per tile, the window's centre is summed as it passes, and the
// next tile's dy is loaded after the store (x's commit and analysis cover
// its latency); at three waves with the filters in registers it spilled and
// ran twice as long.
template <int K, int LT, int TH, int TW, int NT, typename T>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(
    tile_bwd1_waves<GeoTileTrim<K, LT, TH, TW, NT>>()))) void k_tile_bwd1(
    const T* __restrict__ x, const T* __restrict__ dy, const T* __restrict__ wb,
    const T* __restrict__ sb, const T* __restrict__ ww, const T* __restrict__ sw,
    const float* __restrict__ deep, T* __restrict__ dx, float* __restrict__ part,
    float* __restrict__ px, int B, int C, int Hp, int Wp, int upw, int npart) {
    using G = GeoTileTrim<K, LT, TH, TW, NT>;
    using FX = Fetch<G, T, false>;  // x: the tile's core
    using FD = Fetch<G, T, true>;   // dy: the core and its halos
    constexpr int KK = G::KK, Q = G::Q, R = G::R;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    const int c = blockIdx.x % C;
    const int chunk = blockIdx.x / C;
    const int ntx = cdiv(Wp, TW), nty = cdiv(Hp, TH);
    const int units = B * nty * ntx;
    const int u0 = chunk * upw;
    const int u1 = min(u0 + upw, units);
    TileCursor cu = TileCursor::at(u0, B, nty, ntx);  // c stays 0: one channel
    FX fx;
    FD fd;
    if (u0 < u1) {
        fx.issue_tile_buf(x, cu.b, B, C, c, tid, cu.ty * TH, cu.tx * TW, Hp, Wp);
        fd.issue_tile_buf(dy, cu.b, B, C, c, tid, cu.ty * TH, cu.tx * TW, Hp, Wp);
    }
    const Job job = decode_job<G>(tid);
    const int wsrc = job.lvl == 0 ? 0 : KK * (1 + (job.lvl - 1) * 4 + job.s);
    const int win = window_index<G>(job);
    const int pitch = level_pitch<G>(job.lvl);
    const int hrows = by_level<G>(job.lvl, [](auto lc) { return G::hl(decltype(lc)::value); });
    const int wcols = by_level<G>(job.lvl, [](auto lc) { return G::wl(decltype(lc)::value); });
    const int nrows = min(Q, hrows - job.grp * Q);
    const int ncols = min(R, wcols - job.strip * R);
    const bool full = nrows == Q && ncols == R;
    const int dst = win + G::p * pitch + G::p;
    // the folded filters (one channel per workgroup) stay after the arrays;
    // a lane reloads its K x K into registers for each tile's conv, so that
    // they are not live through the store phase beside the next tile's loads
    float* const wl = lds + G::side + wsrc;
    fold_weights<G, T, true>(lds + G::side, wb, wb, sb, ww, sw, C, c, tid);
    for (int i = tid; i < G::side; i += NT) lds[i] = 0.f;
    __syncthreads();
    float gacc[KK];  // rotated: gacc[KK - 1 - t] accumulates tap t
#pragma unroll
    for (int t = 0; t < KK; ++t) gacc[t] = 0.f;
    float sdy = 0.f;

    // the first loads, so that no path into the loop carries loads whose
    // wait would fall behind stores (drain_vmem)
    drain_vmem();
    for (int u = u0; u < u1; ++u) {
        int t = tid;
        const int b = cu.b, y0 = cu.ty * TH, x0 = cu.tx * TW;
        const TileCursor nx = cu.next(B, nty, ntx);
        wave_prio<PrioTileBwd1::commit_x>();
        fx.template commit<true, false>(lds, t);
        // the deeper levels' contribution, in flight through x's analysis
        // (fetched after the dy analysis it was waited for at once, before
        // the conv)
        DeepRegs<G> dr;
        if (deep) fetch_deep<G>(dr, deep, b, C, c, y0, x0, Hp, Wp, t);
        __syncthreads();
        static_for<FX::LEVELS + 1, LT + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, t);
            __syncthreads();
        });
        float ux[Q][R];
        if (job.on)
#pragma unroll
            for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const float v = lds[dst + qq * pitch + j];
                    ux[qq][j] = (full || (qq < nrows && j < ncols)) ? v : 0.f;
                }
        // the core of U^LT_LL(x): the tile's share of the box sums that the
        // deeper levels' weight gradient starts from, held until the tile's
        // stores (stored here, it left a store pending through dy's commit
        // and the conv: their waits for loads then waited for it, and for
        // the deeper levels' fetch right after its issue)
        constexpr int pxh = G::hl(LT), pxw = G::wl(LT);
        const bool pxon = px && t < pxh * pxw && (y0 >> LT) + t / pxw < (Hp >> LT) &&
                          (x0 >> LT) + t % pxw < (Wp >> LT);
        const float pxv = pxon ? lds[G::uidx(LT, 0, 0, t / pxw, t % pxw)] : 0.f;
        __syncthreads();
        wave_prio<PrioTileBwd1::commit_dy>();
        fd.template commit<true, false>(lds, t);
        __syncthreads();
        static_for<FD::LEVELS + 1, LT + 1>([&](auto lc) {
            analysis_level<G, decltype(lc)::value, false>(lds, t);
            __syncthreads();
        });
        float acc[Q][R];
        if (job.on) {
            // the window's centre past the job's part of the core is halo
            // (real neighbours): masked out of the dy sum
            float csum = 0.f;
            float w[KK];
#pragma unroll
            for (int tt = 0; tt < KK; ++tt) w[tt] = wl[tt];
            wave_prio<PrioTileBwd1::conv>();
            conv_corr_tile_csum<K, Q, R>(lds + win, pitch, w, ux, acc, gacc, csum, nrows, ncols);
            wave_prio<PrioTileBwd1::store>();
            if (job.lvl == 0) sdy += csum;
        }
        // the next tile's x after the FMAs, its dy after the store; both
        // unconditional (past the range they cover an empty buffer range:
        // b = B)
        asm volatile("" : "+v"(t));
        const bool more = u + 1 < u1;
        fx.issue_tile_buf(x, more ? nx.b : B, B, C, c, t, nx.ty * TH, nx.tx * TW, Hp, Wp);
        __syncthreads();
        if (job.on) {
#pragma unroll
            for (int qq = 0; qq < Q; ++qq)
#pragma unroll
                for (int j = 0; j < R; ++j)
                    if (full || (qq < nrows && j < ncols)) lds[dst + qq * pitch + j] = acc[qq][j];
        }
        __syncthreads();
        if (deep) {
            add_deep<G>(lds, dr, t);
            __syncthreads();
        }
        static_for<0, LT - 2>([&](auto lc) {
            cascade_level<G, LT - decltype(lc)::value>(lds, t);
            __syncthreads();
        });
        drain_vmem();  // (the next dy is loaded after the store, by design)
        if (pxon) {
            const int hd = Hp >> LT, wd = Wp >> LT;
            const int gy = (y0 >> LT) + t / pxw, gx = (x0 >> LT) + t % pxw;
            px[(size_t(b) * C + c) * hd * wd + size_t(gy) * wd + gx] = pxv;
        }
        final_store<G, T>(lds, dx, b, B, C, c, t, y0, x0, Hp, Wp);
        asm volatile("" : "+v"(t));
        fd.issue_tile_buf(dy, more ? nx.b : B, B, C, c, t, nx.ty * TH, nx.tx * TW, Hp, Wp);
        cu = nx;
        __syncthreads();
    }
    float g[KK];
#pragma unroll
    for (int t = 0; t < KK; ++t) g[t] = gacc[KK - 1 - t];
    reduce_row<G>(lds, g, sdy, part + (size_t(chunk) * C + c) * npart, npart, tid);
}

}  // namespace dev
}  // namespace wtc
