// Zero extension and cropping of NCHW planes, for sides that are not a
// multiple of 2^L (or that no kernel takes directly).  Appending zero rows
// and columns at the end of a plane, running the operator on the larger
// plane and cropping the result gives the operator whose analysis pads an odd
// grid with one zero row (column) at its end at every level: a block that
// lies entirely in the appended zeros has zero coefficients, so every level's
// grid is the per-level grid extended by zeros, and a coefficient past the
// per-level grid only reaches outputs past the image.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_internal.h"

namespace wtc {
namespace {

// dst (planes x Hd x Wd) from src (planes x Hs x Ws): dst[i][j] = src[i][j]
// where i < Hs and j < Ws, else 0.  A thread writes V consecutive elements
// of one destination row (V = 4 when Wd is a multiple of 4, so that the
// write is one 16-byte store for fp32, one 8-byte store for fp16; else 1)
// and reads its source elements one by one (source rows are aligned to no
// more than one element).  The row of a group is found once per group, with
// 32-bit arithmetic where the rows fit it.
template <typename T, int V>
__global__ __launch_bounds__(256) void k_copy_planes(const T* __restrict__ src,
                                                     T* __restrict__ dst, long rows, int Hs,
                                                     int Ws, int Hd, int Wd) {
    const int gpr = Wd / V;  // groups per destination row
    const long groups = rows * gpr;
    for (long g = long(blockIdx.x) * blockDim.x + threadIdx.x; g < groups;
         g += long(gridDim.x) * blockDim.x) {
        long row;
        int j0;
        if (groups < (1L << 31)) {
            const unsigned gu = unsigned(g);
            row = gu / unsigned(gpr);
            j0 = int(gu - unsigned(row) * unsigned(gpr)) * V;
        } else {
            row = g / gpr;
            j0 = int(g - row * gpr) * V;
        }
        long pl;
        int i;
        if (rows < (1L << 31)) {
            const unsigned ru = unsigned(row);
            pl = ru / unsigned(Hd);
            i = int(ru - unsigned(pl) * unsigned(Hd));
        } else {
            pl = row / Hd;
            i = int(row - pl * Hd);
        }
        const T* s = src + (size_t(pl) * Hs + i) * Ws;
        T v[V];
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = (i < Hs && j0 + e < Ws) ? s[j0 + e] : T(0.f);
        T* d = dst + size_t(row) * Wd + j0;
        if constexpr (V == 4) {
            struct alignas(4 * sizeof(T)) Q { T e[4]; };
            *reinterpret_cast<Q*>(d) = Q{{v[0], v[1], v[2], v[3]}};
        } else {
            d[0] = v[0];
        }
    }
}

template <typename T>
hipError_t launch_copy(const void* src, void* dst, long planes, int Hs, int Ws, int Hd, int Wd,
                       hipStream_t stream) {
    const long rows = planes * Hd;
    const bool v4 = Wd % 4 == 0;
    const size_t n = size_t(rows) * (v4 ? Wd / 4 : Wd);
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (v4)
        hipLaunchKernelGGL((k_copy_planes<T, 4>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(src), static_cast<T*>(dst), rows, Hs, Ws, Hd, Wd);
    else
        hipLaunchKernelGGL((k_copy_planes<T, 1>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(src), static_cast<T*>(dst), rows, Hs, Ws, Hd, Wd);
    return hipGetLastError();
}

}  // namespace

hipError_t copy_planes(const void* src, void* dst, long planes, int Hs, int Ws, int Hd, int Wd,
                       int dtype, hipStream_t stream) {
    return dtype == WTCONV_F32 ? launch_copy<float>(src, dst, planes, Hs, Ws, Hd, Wd, stream)
                               : launch_copy<__half>(src, dst, planes, Hs, Ws, Hd, Wd, stream);
}

}  // namespace wtc
