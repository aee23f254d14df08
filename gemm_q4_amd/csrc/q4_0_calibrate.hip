// Measurement aids of the benchmark harness.
//
// mfma_loop_kernel: the sustained rate of the prefill kernel's matrix
// instruction, v_mfma_f32_32x32x16_f16, issued back to back by one wave per
// SIMD on every compute unit.  Under a sustained matrix load this part runs
// below its boost clock, so the harness states the prefill kernel's MFMA
// utilisation against both the published peak and this measured loop rate.
//
// stream_read_kernel: the read rate a plain streaming kernel reaches for a
// given size (each byte read once, 16-byte non-temporal loads, the access the
// small-n kernels make to the weights), and with nothing to read, the cost of
// one launch.  The harness states the small-n kernels' rate against the
// published HBM peak and against this attainable rate for the same bytes.
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

constexpr int kReadThreads = 256;
constexpr int kReadInFlight = 8;   // loads each thread keeps in flight

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u4_t *__restrict__ src,
                                                                  int64_t items,
                                                                  float *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * kReadThreads + threadIdx.x; base < items;
         base += kReadInFlight * stride) {
        u4_t v[kReadInFlight];
#pragma unroll
        for (int u = 0; u < kReadInFlight; ++u) {
            const int64_t i = base + u * stride;
            v[u] = i < items ? __builtin_nontemporal_load(src + i) : u4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    __shared__ uint32_t wacc[kReadThreads / 64];
    if ((threadIdx.x & 63) == 0) wacc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kReadThreads / 64; ++w) s ^= wacc[w];
        // a finite float whatever the bits: the low 23 bits as a fraction
        sink[blockIdx.x] = (float)(s & 0x7fffffu);
    }
}

}  // namespace

hipError_t launch_stream_read(const void *src, int64_t bytes, float *sink, int64_t workgroups,
                              hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0,
                       stream, (const u4_t *)src, bytes / 16, sink);
    return hipGetLastError();
}

int64_t mfma_loop_flops(int64_t workgroups, int64_t iters) {
    return workgroups * 4 * iters * kCalAccs * (int64_t)(2 * 32 * 32 * 16);
}

hipError_t launch_mfma_loop(float *sink, int64_t workgroups, int64_t iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, sink,
                       iters);
    return hipGetLastError();
}

}  // namespace q4
