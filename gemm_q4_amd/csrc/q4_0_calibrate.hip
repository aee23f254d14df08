// Measurement aid of the benchmark harness: the sustained rate of the prefill
// kernel's matrix instruction, v_mfma_f32_32x32x16_f16, issued back to back
// by one wave per SIMD on every compute unit.  The pages report MFMA
// utilisation of the large-n kernel; under a sustained matrix load this part
// runs below its boost clock, so the harness states utilisation against both
// the published peak and this measured loop rate.
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

namespace {

constexpr int kCalAccs = 8;   // independent accumulators: no issue stalls

__global__ __launch_bounds__(256, 1) void mfma_loop_kernel(float *sink, int64_t iters) {
    typedef float f16x_t __attribute__((ext_vector_type(16)));
    const int lane = threadIdx.x & 63;
    h8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.0009765625f * (float)((lane + i) & 15));
        b[i] = (_Float16)(0.0009765625f * (float)((lane * 3 + i) & 15));
    }
    f16x_t acc[kCalAccs];
#pragma unroll
    for (int j = 0; j < kCalAccs; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kCalAccs; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kCalAccs; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

int64_t mfma_loop_flops(int64_t workgroups, int64_t iters) {
    return workgroups * 4 * iters * kCalAccs * (int64_t)(2 * 32 * 32 * 16);
}

hipError_t launch_mfma_loop(float *sink, int64_t workgroups, int64_t iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, sink,
                       iters);
    return hipGetLastError();
}

}  // namespace q4
