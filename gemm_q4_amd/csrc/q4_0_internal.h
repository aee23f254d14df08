// Internal declarations shared by the kernel files and the C-ABI front end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_0_layout.h"

namespace q4 {

// Grid size for a grid-stride loop over `total` items: enough blocks to fill
// the device many times over, capped so the dispatch stays far below the
// 32-bit work-item limit.
inline int64_t grid_for(int64_t total, int block) {
    int64_t g = (total + block - 1) / block;
    const int64_t cap = 1 << 16;
    return g < 1 ? 1 : (g > cap ? cap : g);
}

// Largest workspace a call may need (the caller's buffer, Q4_0_WORKSPACE_MAX):
// per-slice partial sums written by a product kernel and read by the
// reduction kernel that follows it on the same stream, activations converted
// by a pre-pass, routing tables.  Plans that would need more are unsupported.
constexpr size_t kWorkspaceBytes = size_t(128) << 20;

// Compute units and dies (XCDs) of the current HIP device, read once per
// device with hipDeviceGetAttribute.  They set how work is split (and so the
// workspace a call needs).  Without a visible device (size queries on a host
// with no GPU) the MI355X's 256 and 8.
struct DeviceShape {
    int cus, dies;
};
DeviceShape device_shape();

hipError_t launch_repack(const void *blocks, void *packed, int64_t out, int64_t in,
                         hipStream_t stream);
hipError_t launch_unpack(const void *packed, void *blocks, int64_t out, int64_t in,
                         hipStream_t stream);

// Small-n VALU kernel: x staged in LDS as float32, one 16-row tile pair per
// workgroup, four waves splitting K, DPP/shuffle reduction across lanes.
bool gemv_dpp_supports(int64_t n, int64_t out, int64_t in, int x_f16);
hipError_t launch_gemv_dpp(const void *packed, const void *x, int x_f16, float *y,
                           int64_t n, int64_t out, int64_t in, hipStream_t stream);

// Small-n MFMA kernel: activations split into binary16 high and low parts
// (a 16-row MFMA A operand), weights decoded to exact q - 8 in binary16.
// One launch can carry up to kMaxGroupLinears linears that share n and the
// activation type; the workspace holds their K-split partial sums one after
// another (each linear's share is gemv_mfma_workspace_bytes).
constexpr int kMaxGroupLinears = 8;
// rows of x one small-n launch carries; more rows run as row slices
constexpr int64_t kGemvLaunchRows = 64;
struct GemvProblem {
    const void *packed;
    const void *x;
    float *y;
    int64_t out, in;
};
bool gemv_mfma_supports(int64_t n, int64_t out, int64_t in, int x_f16);
size_t gemv_mfma_workspace_bytes(int64_t n, int64_t out, int64_t in);
// Whether one launch can carry these linears together: they agree on the
// rows per launch and on converting x by a pre-pass for every row slice of an
// n-row call.
// Rows per launch for a group of linears (32 or 64: the smallest any of
// them takes alone).
int64_t gemv_mfma_launch_rows(const GemvProblem *probs, int count);
bool gemv_mfma_group_uniform(const GemvProblem *probs, int count, int64_t n);
// Routed small-n product (mixture of experts, by column): y row p = x row
// p / k times the transpose of expert route[p] of a stack of n_experts
// repacked [out x in] matrices; every pair in one launch.
bool gemv_mfma_routed_supports(int64_t pairs, int64_t out, int64_t in);
size_t gemv_mfma_routed_workspace_bytes(int64_t pairs, int64_t out, int64_t in);
hipError_t launch_gemv_mfma_routed(const void *experts, int64_t n_experts, const void *x,
                                   int x_f16, const int32_t *route, int64_t k, float *y,
                                   int64_t n, int64_t out, int64_t in, void *ws,
                                   hipStream_t stream);
// By expert: the pairs routed to each expert are bucketed on the device into
// chunks of 8 rows, each chunk one prepared 8-row product with its expert.
size_t gemv_mfma_by_expert_workspace_bytes(int64_t n, int64_t k, int64_t n_experts, int64_t out,
                                           int64_t in);
bool gemv_mfma_by_expert_supports(int64_t n, int64_t k, int64_t n_experts, int64_t out,
                                  int64_t in);
hipError_t launch_gemv_mfma_by_expert(const void *experts, int64_t n_experts, const void *x,
                                      int x_f16, const int32_t *route, int64_t k, float *y,
                                      int64_t n, int64_t out, int64_t in, void *ws,
                                      hipStream_t stream);
hipError_t launch_gemv_mfma(const void *packed, const void *x, int x_f16, float *y,
                            int64_t n, int64_t out, int64_t in, void *ws,
                            hipStream_t stream);
hipError_t launch_gemv_mfma_group(const GemvProblem *probs, int count, int64_t n, int x_f16,
                                  void *ws, hipStream_t stream);
// y (which may be null: not stored) and, per row t of y, its largest value
// and that value's smallest index, computed in the product's epilogue.
size_t gemv_mfma_argmax_workspace_bytes(int64_t n, int64_t out, int64_t in);
hipError_t launch_gemv_mfma_argmax(const void *packed, const void *x, int x_f16, float *y,
                                   int64_t n, int64_t out, int64_t in, float *max_val,
                                   int32_t *max_idx, void *ws, hipStream_t stream);

// W4A8: activations quantized per 32-value block to int8 (q, d), product on
// the integer matrix cores with the offset-8 correction; n <= 64 (16-row
// launches).
hipError_t launch_quantize_x8(const void *x, int x_f16, int8_t *q, float *d, int64_t n,
                              int64_t in, hipStream_t stream);
bool w4a8_supports(int64_t n, int64_t out, int64_t in);
size_t w4a8_workspace_bytes(int64_t n, int64_t out, int64_t in);
hipError_t launch_gemv_w4a8(const void *packed, const int8_t *q, const float *d, float *y,
                            int64_t n, int64_t out, int64_t in, void *ws, hipStream_t stream);

// Prefill kernel: binary16 MFMA on d * (q - 8) rounded to binary16.  When the
// tiles cannot fill the device it splits K and needs the workspace.
bool gemm_supports(int64_t n, int64_t out, int64_t in, int x_f16);
size_t gemm_workspace_bytes(int64_t n, int64_t out, int64_t in);
hipError_t launch_gemm(const void *packed, const void *x, int x_f16, float *y,
                       int64_t n, int64_t out, int64_t in, void *ws, hipStream_t stream);

// Measurement aids: back-to-back v_mfma_f32_32x32x16_f16 on every SIMD; a
// plain streaming read of `bytes` bytes (an empty launch for 0).
int64_t mfma_loop_flops(int64_t workgroups, int64_t iters);
hipError_t launch_mfma_loop(float *sink, int64_t workgroups, int64_t iters, hipStream_t stream);
hipError_t launch_stream_read(const void *src, int64_t bytes, float *sink, int64_t workgroups,
                              hipStream_t stream);

}  // namespace q4
