// C ABI of libq4_0 (declared in include/q4_0.h): argument checks, kernel
// choice, launches.  Every check runs on the host before any HIP call, so an
// invalid call enqueues nothing and is testable without a GPU.
#include <map>
#include <mutex>
#include <utility>

#include "q4_0.h"
#include "q4_0_internal.h"

namespace {

// Workspaces for K-split kernels, one per (device, stream), allocated on first
// use, so that concurrent calls on different streams never share partial sums.
std::mutex g_ws_mu;
std::map<std::pair<int, uintptr_t>, void *> g_ws;

int get_workspace(hipStream_t stream, void **ws) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return Q4_0_EHIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    const auto key = std::make_pair(dev, (uintptr_t)stream);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
        *ws = it->second;
        return Q4_0_OK;
    }
    void *p = nullptr;
    if (hipMalloc(&p, q4::kWorkspaceBytes) != hipSuccess) return Q4_0_EHIP;
    g_ws[key] = p;
    *ws = p;
    return Q4_0_OK;
}

int check_shape(int64_t n, int64_t out, int64_t in) {
    if (n < 1 || n > Q4_0_MAX_N) return Q4_0_ESHAPE;
    if (out < 1 || out > Q4_0_MAX_OUT) return Q4_0_ESHAPE;
    if (in < 32 || in > Q4_0_MAX_IN || in % 32 != 0) return Q4_0_ESHAPE;
    return Q4_0_OK;
}

bool overlaps(const void *a, size_t alen, const void *b, size_t blen) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + blen && b0 < a0 + alen;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t elem_bytes(int dtype) { return dtype == Q4_0_F16 ? 2 : 4; }

bool supports(int kernel, int64_t n, int64_t out, int64_t in, int x_f16) {
    switch (kernel) {
    case Q4_0_KERNEL_GEMV_DPP: return q4::gemv_dpp_supports(n, out, in, x_f16);
    case Q4_0_KERNEL_GEMV_MFMA: return q4::gemv_mfma_supports(n, out, in, x_f16);
    case Q4_0_KERNEL_GEMM: return q4::gemm_supports(n, out, in, x_f16);
    default: return false;
    }
}

// The automatic choice (goinfer primer ch. 10, "Which kernel runs is a
// runtime decision": pick what is fastest here, not merely what can run).
// Measured on MI355X for n <= 8 over the decode shapes (1024..151936 rows,
// 1024..9728 columns): the MFMA kernel is as fast as or faster than the VALU
// kernel everywhere, so it is first; the VALU kernel takes what it cannot.
// Between decode and prefill (golem README, "Reading a prompt on the card":
// mat-vec up to 16 columns, tiled products from 32): FFN-up 9728 x 2560 at
// n = 9..16 runs in 11.1-11.7 us on the small-n kernel against 26.7-29.6 us
// on the tiled product; with 32-row launches (two 16-row A groups sharing
// each decoded weight fragment) n = 24/32 take 12.8/13.4 us against 32 us,
// and two launches stay ahead up to the kernel's 64 rows (n = 40/48/64:
// 23.4/24.6/26.9 us against 33.5/33.6/35.0 us).
constexpr int64_t kSmallNMax = 64;
// Routed products (golem-server README, "On the card": a column reads the
// matrices it was routed to, a prompt reads each expert once for the columns
// that chose it, the two crossing near thirty-two columns): by expert from
// this many x rows, by column below.  Measured on MI355X (128 experts of 768 x
// 2048, 8 per row, graph replay), by column against by expert: n = 4 8.1 /
// 14.5 us, n = 8 14.6 / 19.1, n = 16 22.6 / 26.2, n = 24 33.3 / 28.4, n = 32
// 39.6 / 29.1, n = 64 69.7 / 36.6: the crossover sits near 24 rows on this part.
constexpr int64_t kByExpertMinN = 24;
int auto_kernel(int64_t n, int64_t out, int64_t in, int x_f16) {
    if (n <= kSmallNMax && q4::gemv_mfma_supports(n, out, in, x_f16))
        return Q4_0_KERNEL_GEMV_MFMA;
    if (n <= 8 && q4::gemv_dpp_supports(n, out, in, x_f16)) return Q4_0_KERNEL_GEMV_DPP;
    return Q4_0_KERNEL_GEMM;
}

int map_hip(hipError_t e) { return e == hipSuccess ? Q4_0_OK : Q4_0_EHIP; }

}  // namespace

extern "C" {

size_t q4_0_blocks_bytes(int64_t out, int64_t in) {
    if (check_shape(1, out, in) != Q4_0_OK) return 0;
    return (size_t)out * (size_t)(in / 32) * 18u;
}

size_t q4_0_packed_bytes(int64_t out, int64_t in) {
    if (check_shape(1, out, in) != Q4_0_OK) return 0;
    return (size_t)q4::Layout(out, in).total_bytes();
}

int q4_0_repack(const void *blocks, void *packed, int64_t out, int64_t in, void *stream) {
    const int st = check_shape(1, out, in);
    if (st != Q4_0_OK) return st;
    if (!blocks || !packed) return Q4_0_ENULL;
    if (!aligned(packed, 16)) return Q4_0_EALIGN;
    if (overlaps(blocks, q4_0_blocks_bytes(out, in), packed, q4_0_packed_bytes(out, in)))
        return Q4_0_EALIAS;
    return map_hip(q4::launch_repack(blocks, packed, out, in, (hipStream_t)stream));
}

int q4_0_unpack(const void *packed, void *blocks, int64_t out, int64_t in, void *stream) {
    const int st = check_shape(1, out, in);
    if (st != Q4_0_OK) return st;
    if (!blocks || !packed) return Q4_0_ENULL;
    if (!aligned(packed, 16)) return Q4_0_EALIGN;
    if (overlaps(blocks, q4_0_blocks_bytes(out, in), packed, q4_0_packed_bytes(out, in)))
        return Q4_0_EALIAS;
    return map_hip(q4::launch_unpack(packed, blocks, out, in, (hipStream_t)stream));
}

int q4_0_kernel_supports(int kernel, int64_t n, int64_t out, int64_t in, int x_dtype) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    if (kernel == Q4_0_KERNEL_AUTO) return Q4_0_OK;
    if (kernel < Q4_0_KERNEL_GEMV_DPP || kernel > Q4_0_KERNEL_GEMM) return Q4_0_EINVAL;
    return supports(kernel, n, out, in, x_dtype == Q4_0_F16) ? Q4_0_OK : Q4_0_EUNSUPPORTED;
}

int q4_0_select_kernel(int64_t n, int64_t out, int64_t in, int x_dtype) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    return auto_kernel(n, out, in, x_dtype == Q4_0_F16);
}

int q4_0_matmul_ex(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                   int64_t out, int64_t in, int kernel, void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    if (kernel < Q4_0_KERNEL_AUTO || kernel > Q4_0_KERNEL_GEMM) return Q4_0_EINVAL;
    if (!packed || !x || !y) return Q4_0_ENULL;
    if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_0_EALIGN;
    const size_t ybytes = (size_t)n * (size_t)out * 4u;
    const size_t xbytes = (size_t)n * (size_t)in * (size_t)elem_bytes(x_dtype);
    if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, packed, q4_0_packed_bytes(out, in)))
        return Q4_0_EALIAS;
    const int x_f16 = x_dtype == Q4_0_F16;
    const int k = kernel == Q4_0_KERNEL_AUTO ? auto_kernel(n, out, in, x_f16) : kernel;
    if (!supports(k, n, out, in, x_f16)) return Q4_0_EUNSUPPORTED;
    const hipStream_t s = (hipStream_t)stream;
    switch (k) {
    case Q4_0_KERNEL_GEMV_DPP: return map_hip(q4::launch_gemv_dpp(packed, x, x_f16, y, n, out, in, s));
    case Q4_0_KERNEL_GEMV_MFMA: {
        void *ws = nullptr;
        if (q4::gemv_mfma_workspace_bytes(n, out, in) > 0) {
            const int wst = get_workspace(s, &ws);
            if (wst != Q4_0_OK) return wst;
        }
        return map_hip(q4::launch_gemv_mfma(packed, x, x_f16, y, n, out, in, ws, s));
    }
    default: {
        void *ws = nullptr;
        if (q4::gemm_workspace_bytes(n, out, in) > 0) {
            const int wst = get_workspace(s, &ws);
            if (wst != Q4_0_OK) return wst;
        }
        return map_hip(q4::launch_gemm(packed, x, x_f16, y, n, out, in, ws, s));
    }
    }
}

int q4_0_matmul(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                int64_t out, int64_t in, void *stream) {
    return q4_0_matmul_ex(packed, x, x_dtype, y, n, out, in, Q4_0_KERNEL_AUTO, stream);
}

int q4_0_matmul_argmax(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                       int64_t out, int64_t in, float *max_val, int32_t *max_idx,
                       void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    if (!packed || !x || !max_val || !max_idx) return Q4_0_ENULL;
    if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(max_val, 4) ||
        !aligned(max_idx, 4))
        return Q4_0_EALIGN;
    const size_t xbytes = (size_t)n * (size_t)in * (size_t)elem_bytes(x_dtype);
    const size_t wbytes = q4_0_packed_bytes(out, in);
    const size_t ybytes = y ? (size_t)n * (size_t)out * 4u : 0;
    const size_t rbytes = (size_t)n * 4u;
    const void *outs[3] = {y, max_val, max_idx};
    const size_t olen[3] = {ybytes, rbytes, rbytes};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], olen[i], x, xbytes) || overlaps(outs[i], olen[i], packed, wbytes))
            return Q4_0_EALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], olen[i], outs[j], olen[j])) return Q4_0_EALIAS;
    }
    const int x_f16 = x_dtype == Q4_0_F16;
    if (!q4::gemv_mfma_supports(n, out, in, x_f16) ||
        q4::gemv_mfma_argmax_workspace_bytes(n, out, in) > q4::kWorkspaceBytes)
        return Q4_0_EUNSUPPORTED;
    const hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    const int wst = get_workspace(s, &ws);
    if (wst != Q4_0_OK) return wst;
    return map_hip(q4::launch_gemv_mfma_argmax(packed, x, x_f16, y, n, out, in, max_val, max_idx,
                                               ws, s));
}

int q4_0_quantize_x8(const void *x, int x_dtype, int8_t *q, float *d, int64_t n, int64_t in,
                     void *stream) {
    const int st = check_shape(n, 1, in);
    if (st != Q4_0_OK) return st;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    if (!x || !q || !d) return Q4_0_ENULL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4)) return Q4_0_EALIGN;
    const size_t xbytes = (size_t)n * (size_t)in * (size_t)elem_bytes(x_dtype);
    const size_t qbytes = (size_t)n * (size_t)in, dbytes = (size_t)n * (size_t)(in / 32) * 4u;
    if (overlaps(q, qbytes, x, xbytes) || overlaps(d, dbytes, x, xbytes) ||
        overlaps(q, qbytes, d, dbytes))
        return Q4_0_EALIAS;
    return map_hip(q4::launch_quantize_x8(x, x_dtype == Q4_0_F16, q, d, n, in,
                                          (hipStream_t)stream));
}

int q4_0_matmul_w4a8(const void *packed, const int8_t *q, const float *d, float *y, int64_t n,
                     int64_t out, int64_t in, void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!packed || !q || !d || !y) return Q4_0_ENULL;
    if (!aligned(packed, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4))
        return Q4_0_EALIGN;
    const size_t ybytes = (size_t)n * (size_t)out * 4u;
    if (overlaps(y, ybytes, packed, q4_0_packed_bytes(out, in)) ||
        overlaps(y, ybytes, q, (size_t)n * (size_t)in) ||
        overlaps(y, ybytes, d, (size_t)n * (size_t)(in / 32) * 4u))
        return Q4_0_EALIAS;
    if (!q4::w4a8_supports(n, out, in)) return Q4_0_EUNSUPPORTED;
    const hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    if (q4::w4a8_workspace_bytes(n, out, in) > 0) {
        const int wst = get_workspace(s, &ws);
        if (wst != Q4_0_OK) return wst;
    }
    return map_hip(q4::launch_gemv_w4a8(packed, q, d, y, n, out, in, ws, s));
}

int q4_0_matmul_routed(const void *experts, int64_t n_experts, const void *x, int x_dtype,
                       const int32_t *route, int64_t k, float *y, int64_t n, int64_t out,
                       int64_t in, void *stream) {
    return q4_0_matmul_routed_ex(experts, n_experts, x, x_dtype, route, k, y, n, out, in,
                                 Q4_0_ROUTE_AUTO, stream);
}

int q4_0_select_route(int64_t n, int64_t k, int64_t n_experts, int64_t out, int64_t in) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (n_experts < 1 || n_experts > Q4_0_MAX_EXPERTS || k < 1 || k > Q4_0_MAX_ROUTED)
        return Q4_0_EINVAL;
    const bool col = q4::gemv_mfma_routed_supports(n * k, out, in);
    const bool exp = q4::gemv_mfma_by_expert_supports(n, k, n_experts, out, in);
    if (exp && (n >= kByExpertMinN || !col)) return Q4_0_ROUTE_BY_EXPERT;
    if (col) return Q4_0_ROUTE_BY_COLUMN;
    return Q4_0_EUNSUPPORTED;
}

int q4_0_matmul_routed_ex(const void *experts, int64_t n_experts, const void *x, int x_dtype,
                          const int32_t *route, int64_t k, float *y, int64_t n, int64_t out,
                          int64_t in, int route_kernel, void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    if (route_kernel != Q4_0_ROUTE_AUTO && route_kernel != Q4_0_ROUTE_BY_COLUMN &&
        route_kernel != Q4_0_ROUTE_BY_EXPERT)
        return Q4_0_EINVAL;
    if (n_experts < 1 || n_experts > Q4_0_MAX_EXPERTS || k < 1 || k > Q4_0_MAX_ROUTED)
        return Q4_0_EINVAL;
    if (!experts || !x || !route || !y) return Q4_0_ENULL;
    if (!aligned(experts, 16) || !aligned(x, 16) || !aligned(route, 4) || !aligned(y, 4))
        return Q4_0_EALIGN;
    const int64_t pairs = n * k;
    const size_t ybytes = (size_t)pairs * (size_t)out * 4u;
    const size_t xbytes = (size_t)n * (size_t)in * (size_t)elem_bytes(x_dtype);
    const size_t wbytes = (size_t)n_experts * q4_0_packed_bytes(out, in);
    if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, experts, wbytes) ||
        overlaps(y, ybytes, route, (size_t)pairs * 4u))
        return Q4_0_EALIAS;
    int rk = route_kernel;
    if (rk == Q4_0_ROUTE_AUTO) {
        rk = q4_0_select_route(n, k, n_experts, out, in);
        if (rk < 0) return rk;
    } else if (rk == Q4_0_ROUTE_BY_COLUMN ? !q4::gemv_mfma_routed_supports(pairs, out, in)
                                          : !q4::gemv_mfma_by_expert_supports(n, k, n_experts,
                                                                              out, in)) {
        return Q4_0_EUNSUPPORTED;
    }
    const hipStream_t s = (hipStream_t)stream;
    const size_t wsb = rk == Q4_0_ROUTE_BY_COLUMN
                           ? q4::gemv_mfma_routed_workspace_bytes(pairs, out, in)
                           : q4::gemv_mfma_by_expert_workspace_bytes(n, k, n_experts, out, in);
    void *ws = nullptr;
    if (wsb > 0) {
        const int wst = get_workspace(s, &ws);
        if (wst != Q4_0_OK) return wst;
    }
    const int f16 = x_dtype == Q4_0_F16;
    return map_hip(rk == Q4_0_ROUTE_BY_COLUMN
                       ? q4::launch_gemv_mfma_routed(experts, n_experts, x, f16, route, k, y, n,
                                                     out, in, ws, s)
                       : q4::launch_gemv_mfma_by_expert(experts, n_experts, x, f16, route, k, y,
                                                        n, out, in, ws, s));
}

int q4_0_matmul_grouped(const q4_0_linear *linears, int count, int x_dtype, int64_t n,
                        void *stream) {
    if (!linears) return Q4_0_ENULL;
    if (count < 1 || count > Q4_0_MAX_GROUP) return Q4_0_EINVAL;
    if (x_dtype != Q4_0_F32 && x_dtype != Q4_0_F16) return Q4_0_EINVAL;
    const int x_f16 = x_dtype == Q4_0_F16;
    bool one_launch = true;
    size_t ws_total = 0;
    q4::GemvProblem probs[Q4_0_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        const q4_0_linear &L = linears[i];
        const int st = check_shape(n, L.out, L.in);
        if (st != Q4_0_OK) return st;
        if (!L.packed || !L.x || !L.y) return Q4_0_ENULL;
        if (!aligned(L.packed, 16) || !aligned(L.x, 16) || !aligned(L.y, 4)) return Q4_0_EALIGN;
        const size_t ybytes = (size_t)n * (size_t)L.out * 4u;
        for (int j = 0; j < count; ++j) {
            const q4_0_linear &M = linears[j];
            const size_t xb = (size_t)n * (size_t)M.in * (size_t)elem_bytes(x_dtype);
            if (overlaps(L.y, ybytes, M.x, xb) ||
                overlaps(L.y, ybytes, M.packed, q4_0_packed_bytes(M.out, M.in)))
                return Q4_0_EALIAS;
            if (j != i && overlaps(L.y, ybytes, M.y, (size_t)n * (size_t)M.out * 4u))
                return Q4_0_EALIAS;
        }
        if (auto_kernel(n, L.out, L.in, x_f16) != Q4_0_KERNEL_GEMV_MFMA)
            one_launch = false;
        else
            ws_total += q4::gemv_mfma_workspace_bytes(n, L.out, L.in);
        probs[i] = {L.packed, L.x, L.y, L.out, L.in};
    }
    if (ws_total > q4::kWorkspaceBytes) one_launch = false;
    if (one_launch && !q4::gemv_mfma_group_uniform(probs, count, n)) one_launch = false;
    const hipStream_t s = (hipStream_t)stream;
    if (!one_launch) {
        for (int i = 0; i < count; ++i) {
            const q4_0_linear &L = linears[i];
            const int st = q4_0_matmul(L.packed, L.x, x_dtype, L.y, n, L.out, L.in, stream);
            if (st != Q4_0_OK) return st;
        }
        return Q4_0_OK;
    }
    void *ws = nullptr;
    if (ws_total > 0) {
        const int wst = get_workspace(s, &ws);
        if (wst != Q4_0_OK) return wst;
    }
    // one launch per slice of up to `lr` rows of every x and y
    const int64_t esize = elem_bytes(x_dtype);
    const int64_t lr = q4::gemv_mfma_launch_rows(probs, count);
    for (int64_t r0 = 0; r0 < n; r0 += lr) {
        const int64_t nr = n - r0 < lr ? n - r0 : lr;
        q4::GemvProblem ps[Q4_0_MAX_GROUP];
        for (int i = 0; i < count; ++i)
            ps[i] = {probs[i].packed, (const uint8_t *)probs[i].x + r0 * probs[i].in * esize,
                     probs[i].y + r0 * probs[i].out, probs[i].out, probs[i].in};
        const int st = map_hip(q4::launch_gemv_mfma_group(ps, count, nr, x_f16, ws, s));
        if (st != Q4_0_OK) return st;
    }
    return Q4_0_OK;
}

int q4_0_mfma_loop(float *sink, int64_t workgroups, int64_t iters, int64_t *flops,
                   void *stream) {
    if (!sink || !flops) return Q4_0_ENULL;
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > 1000000) return Q4_0_EINVAL;
    *flops = q4::mfma_loop_flops(workgroups, iters);
    return map_hip(q4::launch_mfma_loop(sink, workgroups, iters, (hipStream_t)stream));
}

const char *q4_0_strerror(int status) {
    switch (status) {
    case Q4_0_OK: return "success";
    case Q4_0_EINVAL: return "invalid dtype or kernel selector";
    case Q4_0_ESHAPE: return "invalid shape (need n, out >= 1, in >= 32, in % 32 == 0, within limits)";
    case Q4_0_ENULL: return "null pointer argument";
    case Q4_0_EALIGN: return "misaligned pointer (packed and x need 16 bytes, y 4 bytes)";
    case Q4_0_EALIAS: return "output buffer overlaps an input buffer";
    case Q4_0_EUNSUPPORTED: return "the requested kernel cannot take this shape";
    case Q4_0_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

int q4_0_version(void) { return 100; }

int q4_0_release_workspaces(void) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    int dev0 = 0;
    if (hipGetDevice(&dev0) != hipSuccess) return Q4_0_EHIP;
    int st = Q4_0_OK;
    for (auto &kv : g_ws) {
        if (hipSetDevice(kv.first.first) != hipSuccess ||
            hipStreamSynchronize((hipStream_t)kv.first.second) != hipSuccess ||
            hipFree(kv.second) != hipSuccess)
            st = Q4_0_EHIP;
    }
    g_ws.clear();
    if (hipSetDevice(dev0) != hipSuccess) st = Q4_0_EHIP;
    return st;
}

}  // extern "C"
