// Issue-rate probe of the vector ALU on the GPU it runs on: a grid of
// independent fp32 multiply-add chains (v_fmac_f32, no packed-FP32
// instructions: this file is built with packed-FP32 selection off like the
// library), and the same with v_dot2c_f32_f16 (two fp16 products added to an
// fp32 sum per lane and instruction).  Prints one JSON line: lane-instructions
// per second and the FLOP rate each implies (2 per fma lane-instruction,
// 4 per dot2 lane-instruction), best of four launches per configuration.
// Used to pick the roof the layer's kernels are measured against.
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kIters = 1000;
constexpr int kUnroll = 8;

template <int KIND, int NCH>
__global__ __launch_bounds__(kThreads) void chains(float* out, float seed) {
    float a[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) a[i] = seed + i + threadIdx.x;
    half2_t h;
    h.x = static_cast<_Float16>(seed * 0.5f);
    h.y = static_cast<_Float16>(seed * 0.25f);
    const float w = seed * 1e-3f, b = seed * 2e-3f;
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
        for (int r = 0; r < kUnroll; ++r)
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                if constexpr (KIND == 0)
                    a[i] = fmaf(w, a[i], b);
                else
                    a[i] = __builtin_amdgcn_fdot2(h, h, a[i], false);
            }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) s += a[i];
    out[size_t(blockIdx.x) * kThreads + threadIdx.x] = s;  // one float per thread of the grid
}

template <int KIND, int NCH>
double rate(float* out, int blocks) {
    hipEvent_t e0, e1;
    hipEventCreate(&e0);
    hipEventCreate(&e1);
    float best = 1e30f;
    for (int rep = 0; rep < 4; ++rep) {
        hipEventRecord(e0);
        hipLaunchKernelGGL((chains<KIND, NCH>), dim3(blocks), dim3(kThreads), 0, 0, out, 1.0f);
        hipEventRecord(e1);
        hipEventSynchronize(e1);
        float ms = 0.f;
        hipEventElapsedTime(&ms, e0, e1);
        if (ms < best) best = ms;
    }
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    const double lane_insts = double(blocks) * kThreads * kIters * kUnroll * NCH;
    return lane_insts / (best * 1e-3);
}

}  // namespace

int main() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        std::fprintf(stderr, "no HIP device\n");
        return 1;
    }
    const int blocks = cus * 8;  // 8 workgroups of 4 waves per compute unit
    float* out = nullptr;
    if (hipMalloc(&out, size_t(blocks) * kThreads * sizeof(float)) != hipSuccess) return 1;
    const double f16 = rate<0, 16>(out, blocks), f32 = rate<0, 32>(out, blocks);
    const double d16 = rate<1, 16>(out, blocks);
    const double fma = f16 > f32 ? f16 : f32;
    std::printf("{\"compute_units\": %d, \"fmac_f32_lane_inst_per_s\": %.4g, \"fmac_f32_tflops\": %.2f, "
                "\"dot2c_f32_f16_lane_inst_per_s\": %.4g, \"dot2c_f32_f16_tflops\": %.2f}\n",
                cus, fma, 2.0 * fma / 1e12, d16, 4.0 * d16 / 1e12);
    hipFree(out);
    return 0;
}
