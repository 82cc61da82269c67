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
// where i < Hs and j < Ws, else 0.  One thread per destination element.
template <typename T>
__global__ __launch_bounds__(256) void k_copy_planes(const T* __restrict__ src,
                                                     T* __restrict__ dst, long planes, int Hs,
                                                     int Ws, int Hd, int Wd) {
    const size_t n = size_t(planes) * Hd * Wd;
    for (size_t e = size_t(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += size_t(gridDim.x) * blockDim.x) {
        const int j = int(e % Wd);
        const size_t r = e / Wd;
        const int i = int(r % Hd);
        const size_t pl = r / Hd;
        T v = T(0.f);
        if (i < Hs && j < Ws) v = src[(pl * Hs + i) * Ws + j];
        dst[e] = v;
    }
}

template <typename T>
hipError_t launch_copy(const void* src, void* dst, long planes, int Hs, int Ws, int Hd, int Wd,
                       hipStream_t stream) {
    const size_t n = size_t(planes) * Hd * Wd;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_copy_planes<T>, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const T*>(src), static_cast<T*>(dst), planes, Hs, Ws, Hd, Wd);
    return hipGetLastError();
}

}  // namespace

hipError_t copy_planes(const void* src, void* dst, long planes, int Hs, int Ws, int Hd, int Wd,
                       int dtype, hipStream_t stream) {
    return dtype == WTCONV_F32 ? launch_copy<float>(src, dst, planes, Hs, Ws, Hd, Wd, stream)
                               : launch_copy<__half>(src, dst, planes, Hs, Ws, Hd, Wd, stream);
}

}  // namespace wtc
