// C ABI of libq4_0 (declared in include/q4_0.h): argument checks, kernel
// choice, workspace sizes, launches.  Every check runs on the host before any
// HIP call, so an invalid call enqueues nothing and is testable without a
// GPU.  The library owns no device memory: scratch comes from the caller.
#include <mutex>

#include "q4_0.h"
#include "q4_0_internal.h"

namespace q4 {

constexpr int kMaxDevices = 64;

namespace {
std::mutex g_shape_mu;
DeviceShape g_shape[kMaxDevices];
bool g_shape_known[kMaxDevices];
}  // namespace

DeviceShape device_shape() {
    const DeviceShape mi355x = {256, 8};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return mi355x;
    }
    std::lock_guard<std::mutex> lock(g_shape_mu);
    if (!g_shape_known[dev]) {
        int cus = 0, dies = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus < 1) {
            (void)hipGetLastError();
            return mi355x;
        }
        if (hipDeviceGetAttribute(&dies, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
            dies < 1 || cus % dies != 0) {
            (void)hipGetLastError();
            dies = 1;
        }
        g_shape[dev] = {cus, dies};
        g_shape_known[dev] = true;
    }
    return g_shape[dev];
}

}  // namespace q4

namespace {

// Scratch of q4_0_matmul_static: one array per GPU (each device holds its own
// copy of a __device__ variable), alive until the process ends.  Host code
// must not use the array's name as an address: the per-device address comes
// from hipGetSymbolAddress, taken once per device on the first call there.
static __device__ __align__(256) uint8_t scratch[Q4_0_STATIC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void *g_scratch_ptr[q4::kMaxDevices];

int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= q4::kMaxDevices) {
        (void)hipGetLastError();
        return Q4_0_EHIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return Q4_0_EHIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return Q4_0_OK;
}

int check_shape(int64_t n, int64_t out, int64_t in) {
    if (n < 1 || n > Q4_0_MAX_N) return Q4_0_ESHAPE;
    if (out < 1 || out > Q4_0_MAX_OUT) return Q4_0_ESHAPE;
    if (in < 32 || in > Q4_0_MAX_IN || in % 32 != 0) return Q4_0_ESHAPE;
    return Q4_0_OK;
}

bool valid_dtype(int d) { return d == Q4_0_F32 || d == Q4_0_F16; }

bool overlaps(const void *a, size_t alen, const void *b, size_t blen) {
    if (!a || !b || alen == 0 || blen == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + blen && b0 < a0 + alen;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t elem_bytes(int dtype) { return dtype == Q4_0_F16 ? 2 : 4; }

// A buffer of the call, for the workspace's overlap check.
struct Span {
    const void *p;
    size_t len;
};

// The workspace of a call that needs `need` bytes: present, large enough,
// aligned, and overlapping none of the call's buffers.
int check_workspace(const void *ws, size_t have, size_t need, const Span *spans, int nspans) {
    if (need == 0) return Q4_0_OK;
    if (!ws || have < need) return Q4_0_EWORKSPACE;
    if (!aligned(ws, Q4_0_WORKSPACE_ALIGN)) return Q4_0_EALIGN;
    for (int i = 0; i < nspans; ++i)
        if (overlaps(ws, need, spans[i].p, spans[i].len)) return Q4_0_EALIAS;
    return Q4_0_OK;
}

bool supports(int kernel, int64_t n, int64_t out, int64_t in, int x_f16) {
    switch (kernel) {
    case Q4_0_KERNEL_GEMV_DPP: return q4::gemv_dpp_supports(n, out, in, x_f16);
    case Q4_0_KERNEL_GEMV_MFMA: return q4::gemv_mfma_supports(n, out, in, x_f16);
    case Q4_0_KERNEL_GEMM: return q4::gemm_supports(n, out, in, x_f16);
    default: return false;
    }
}

size_t kernel_workspace(int kernel, int64_t n, int64_t out, int64_t in) {
    switch (kernel) {
    case Q4_0_KERNEL_GEMV_MFMA: return q4::gemv_mfma_workspace_bytes(n, out, in);
    case Q4_0_KERNEL_GEMM: return q4::gemm_workspace_bytes(n, out, in);
    default: return 0;
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
// Routed products (golem-server README, "On the card": by column or by
// expert, with a crossover that the page places near thirty-two columns on
// its card): by expert from this many x rows, by column below.  Measured on
// MI355X (128 experts of 768 x 2048, 8 per row, graph replay), by column
// against by expert: n = 4 8.1 / 14.5 us, n = 8 14.6 / 19.1, n = 16 22.6 /
// 26.2, n = 24 33.3 / 28.4, n = 32 39.6 / 29.1, n = 64 69.7 / 36.6: the
// crossover sits near 24 rows on this part.
constexpr int64_t kByExpertMinN = 24;
int auto_kernel(int64_t n, int64_t out, int64_t in, int x_f16) {
    if (n <= kSmallNMax && q4::gemv_mfma_supports(n, out, in, x_f16))
        return Q4_0_KERNEL_GEMV_MFMA;
    if (n <= 8 && q4::gemv_dpp_supports(n, out, in, x_f16)) return Q4_0_KERNEL_GEMV_DPP;
    return Q4_0_KERNEL_GEMM;
}

int map_hip(hipError_t e) { return e == hipSuccess ? Q4_0_OK : Q4_0_EHIP; }

// Kernel a q4_0_matmul_ex call runs, after its shape, dtype and selector
// checks, or a negative status.
int resolve_kernel(int64_t n, int64_t out, int64_t in, int x_dtype, int kernel) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
    if (kernel < Q4_0_KERNEL_AUTO || kernel > Q4_0_KERNEL_GEMM) return Q4_0_EINVAL;
    const int x_f16 = x_dtype == Q4_0_F16;
    const int k = kernel == Q4_0_KERNEL_AUTO ? auto_kernel(n, out, in, x_f16) : kernel;
    if (!supports(k, n, out, in, x_f16)) return Q4_0_EUNSUPPORTED;
    return k;
}

int launch_kernel(int k, const void *packed, const void *x, int x_f16, float *y, int64_t n,
                  int64_t out, int64_t in, void *ws, hipStream_t s) {
    switch (k) {
    case Q4_0_KERNEL_GEMV_DPP:
        return map_hip(q4::launch_gemv_dpp(packed, x, x_f16, y, n, out, in, s));
    case Q4_0_KERNEL_GEMV_MFMA:
        return map_hip(q4::launch_gemv_mfma(packed, x, x_f16, y, n, out, in, ws, s));
    default:
        return map_hip(q4::launch_gemm(packed, x, x_f16, y, n, out, in, ws, s));
    }
}

// Checks of one linear of a grouped call (shapes, pointers, overlaps with
// every linear of the group).
int check_linear(const q4_0_linear *linears, int count, int i, int x_dtype, int64_t n) {
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
            overlaps(L.y, ybytes, M.packed, q4::Layout(M.out, M.in).total_bytes()))
            return Q4_0_EALIAS;
        if (j != i && overlaps(L.y, ybytes, M.y, (size_t)n * (size_t)M.out * 4u))
            return Q4_0_EALIAS;
    }
    return Q4_0_OK;
}

// How a grouped call runs: one launch (per row slice) on the small-n MFMA
// kernel, or each linear as q4_0_matmul would; the workspace it needs.
struct GroupPlan {
    bool one_launch;
    size_t ws;
    int kernels[Q4_0_MAX_GROUP];
};

int plan_group(const q4_0_linear *linears, int count, int x_dtype, int64_t n, GroupPlan *gp) {
    if (!linears) return Q4_0_ENULL;
    if (count < 1 || count > Q4_0_MAX_GROUP) return Q4_0_EINVAL;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
    const int x_f16 = x_dtype == Q4_0_F16;
    gp->one_launch = true;
    size_t sum = 0, most = 0;
    q4::GemvProblem probs[Q4_0_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        const q4_0_linear &L = linears[i];
        const int k = resolve_kernel(n, L.out, L.in, x_dtype, Q4_0_KERNEL_AUTO);
        if (k < 0) return k;
        gp->kernels[i] = k;
        const size_t w = kernel_workspace(k, n, L.out, L.in);
        if (w > most) most = w;
        if (k == Q4_0_KERNEL_GEMV_MFMA)
            sum += w;
        else
            gp->one_launch = false;
        probs[i] = {L.packed, L.x, L.y, L.out, L.in};
    }
    (void)x_f16;
    if (sum > q4::kWorkspaceBytes) gp->one_launch = false;
    if (gp->one_launch && !q4::gemv_mfma_group_uniform(probs, count, n)) gp->one_launch = false;
    gp->ws = gp->one_launch ? sum : most;
    return Q4_0_OK;
}

int argmax_workspace(int64_t n, int64_t out, int64_t in, int x_dtype, size_t *bytes) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
    const int x_f16 = x_dtype == Q4_0_F16;
    if (!q4::gemv_mfma_supports(n, out, in, x_f16)) return Q4_0_EUNSUPPORTED;
    const size_t w = q4::gemv_mfma_argmax_workspace_bytes(n, out, in);
    if (w > q4::kWorkspaceBytes) return Q4_0_EUNSUPPORTED;
    *bytes = w;
    return Q4_0_OK;
}

// The routed form a call runs (after its checks), or a negative status.
int routed_form(int64_t n, int64_t k, int64_t n_experts, int64_t out, int64_t in,
                int route_kernel) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (route_kernel != Q4_0_ROUTE_AUTO && route_kernel != Q4_0_ROUTE_BY_COLUMN &&
        route_kernel != Q4_0_ROUTE_BY_EXPERT)
        return Q4_0_EINVAL;
    if (n_experts < 1 || n_experts > Q4_0_MAX_EXPERTS || k < 1 || k > Q4_0_MAX_ROUTED)
        return Q4_0_EINVAL;
    const bool col = q4::gemv_mfma_routed_supports(n * k, out, in);
    const bool exp = q4::gemv_mfma_by_expert_supports(n, k, n_experts, out, in);
    if (route_kernel == Q4_0_ROUTE_AUTO) {
        if (exp && (n >= kByExpertMinN || !col)) return Q4_0_ROUTE_BY_EXPERT;
        if (col) return Q4_0_ROUTE_BY_COLUMN;
        return Q4_0_EUNSUPPORTED;
    }
    if (route_kernel == Q4_0_ROUTE_BY_COLUMN ? !col : !exp) return Q4_0_EUNSUPPORTED;
    return route_kernel;
}

size_t routed_workspace(int form, int64_t n, int64_t k, int64_t n_experts, int64_t out,
                        int64_t in) {
    return form == Q4_0_ROUTE_BY_COLUMN
               ? q4::gemv_mfma_routed_workspace_bytes(n * k, out, in)
               : q4::gemv_mfma_by_expert_workspace_bytes(n, k, n_experts, out, in);
}

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
    const int k = resolve_kernel(n, out, in, x_dtype, kernel);
    return k < 0 ? k : Q4_0_OK;
}

int q4_0_select_kernel(int64_t n, int64_t out, int64_t in, int x_dtype) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
    return auto_kernel(n, out, in, x_dtype == Q4_0_F16);
}

int q4_0_matmul_workspace_size(int64_t n, int64_t out, int64_t in, int x_dtype, int kernel,
                               size_t *bytes) {
    if (!bytes) return Q4_0_ENULL;
    const int k = resolve_kernel(n, out, in, x_dtype, kernel);
    if (k < 0) return k;
    *bytes = kernel_workspace(k, n, out, in);
    return Q4_0_OK;
}

int q4_0_matmul_ex(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                   int64_t out, int64_t in, int kernel, void *workspace,
                   size_t workspace_bytes, void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
    if (kernel < Q4_0_KERNEL_AUTO || kernel > Q4_0_KERNEL_GEMM) return Q4_0_EINVAL;
    if (!packed || !x || !y) return Q4_0_ENULL;
    if (!aligned(packed, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_0_EALIGN;
    const size_t ybytes = (size_t)n * (size_t)out * 4u;
    const size_t xbytes = (size_t)n * (size_t)in * (size_t)elem_bytes(x_dtype);
    const size_t wbytes = q4_0_packed_bytes(out, in);
    if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, packed, wbytes))
        return Q4_0_EALIAS;
    const int k = resolve_kernel(n, out, in, x_dtype, kernel);
    if (k < 0) return k;
    const Span spans[3] = {{packed, wbytes}, {x, xbytes}, {y, ybytes}};
    const int wst = check_workspace(workspace, workspace_bytes,
                                    kernel_workspace(k, n, out, in), spans, 3);
    if (wst != Q4_0_OK) return wst;
    return launch_kernel(k, packed, x, x_dtype == Q4_0_F16, y, n, out, in, workspace,
                         (hipStream_t)stream);
}

int q4_0_matmul(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                int64_t out, int64_t in, void *workspace, size_t workspace_bytes,
                void *stream) {
    return q4_0_matmul_ex(packed, x, x_dtype, y, n, out, in, Q4_0_KERNEL_AUTO, workspace,
                          workspace_bytes, stream);
}

int q4_0_matmul_static(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                       int64_t out, int64_t in, void *stream) {
    // the checks of q4_0_matmul first (nothing is touched on an invalid call),
    // then the scratch need against the static buffer
    size_t need = 0;
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
    if (!packed || !x || !y) return Q4_0_ENULL;
    const int k = resolve_kernel(n, out, in, x_dtype, Q4_0_KERNEL_AUTO);
    if (k < 0) return k;
    need = kernel_workspace(k, n, out, in);
    if (need > (size_t)Q4_0_STATIC_SCRATCH_BYTES) return Q4_0_EWORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        const int sst = scratch_address(&ws);
        if (sst != Q4_0_OK) return sst;
    }
    return q4_0_matmul_ex(packed, x, x_dtype, y, n, out, in, Q4_0_KERNEL_AUTO, ws,
                          need > 0 ? (size_t)Q4_0_STATIC_SCRATCH_BYTES : 0, stream);
}

int q4_0_argmax_workspace_size(int64_t n, int64_t out, int64_t in, int x_dtype,
                               size_t *bytes) {
    if (!bytes) return Q4_0_ENULL;
    return argmax_workspace(n, out, in, x_dtype, bytes);
}

int q4_0_matmul_argmax(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                       int64_t out, int64_t in, float *max_val, int32_t *max_idx,
                       void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
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
    size_t need = 0;
    const int ast = argmax_workspace(n, out, in, x_dtype, &need);
    if (ast != Q4_0_OK) return ast;
    const Span spans[5] = {{packed, wbytes}, {x, xbytes}, {y, ybytes}, {max_val, rbytes},
                           {max_idx, rbytes}};
    const int wst = check_workspace(workspace, workspace_bytes, need, spans, 5);
    if (wst != Q4_0_OK) return wst;
    return map_hip(q4::launch_gemv_mfma_argmax(packed, x, x_dtype == Q4_0_F16, y, n, out, in,
                                               max_val, max_idx, workspace,
                                               (hipStream_t)stream));
}

int q4_0_quantize_x8(const void *x, int x_dtype, int8_t *q, float *d, int64_t n, int64_t in,
                     void *stream) {
    const int st = check_shape(n, 1, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
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

int q4_0_w4a8_workspace_size(int64_t n, int64_t out, int64_t in, size_t *bytes) {
    if (!bytes) return Q4_0_ENULL;
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!q4::w4a8_supports(n, out, in)) return Q4_0_EUNSUPPORTED;
    *bytes = q4::w4a8_workspace_bytes(n, out, in);
    return Q4_0_OK;
}

int q4_0_matmul_w4a8(const void *packed, const int8_t *q, const float *d, float *y, int64_t n,
                     int64_t out, int64_t in, void *workspace, size_t workspace_bytes,
                     void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!packed || !q || !d || !y) return Q4_0_ENULL;
    if (!aligned(packed, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4))
        return Q4_0_EALIGN;
    const size_t ybytes = (size_t)n * (size_t)out * 4u;
    const size_t wbytes = q4_0_packed_bytes(out, in);
    const size_t qbytes = (size_t)n * (size_t)in, dbytes = (size_t)n * (size_t)(in / 32) * 4u;
    if (overlaps(y, ybytes, packed, wbytes) || overlaps(y, ybytes, q, qbytes) ||
        overlaps(y, ybytes, d, dbytes))
        return Q4_0_EALIAS;
    if (!q4::w4a8_supports(n, out, in)) return Q4_0_EUNSUPPORTED;
    const Span spans[4] = {{packed, wbytes}, {q, qbytes}, {d, dbytes}, {y, ybytes}};
    const int wst = check_workspace(workspace, workspace_bytes,
                                    q4::w4a8_workspace_bytes(n, out, in), spans, 4);
    if (wst != Q4_0_OK) return wst;
    return map_hip(q4::launch_gemv_w4a8(packed, q, d, y, n, out, in, workspace,
                                        (hipStream_t)stream));
}

int q4_0_select_route(int64_t n, int64_t k, int64_t n_experts, int64_t out, int64_t in) {
    return routed_form(n, k, n_experts, out, in, Q4_0_ROUTE_AUTO);
}

int q4_0_routed_workspace_size(int64_t n, int64_t k, int64_t n_experts, int64_t out,
                               int64_t in, int route_kernel, size_t *bytes) {
    if (!bytes) return Q4_0_ENULL;
    const int form = routed_form(n, k, n_experts, out, in, route_kernel);
    if (form < 0) return form;
    *bytes = routed_workspace(form, n, k, n_experts, out, in);
    return Q4_0_OK;
}

int q4_0_matmul_routed_ex(const void *experts, int64_t n_experts, const void *x, int x_dtype,
                          const int32_t *route, int64_t k, float *y, int64_t n, int64_t out,
                          int64_t in, int route_kernel, void *workspace,
                          size_t workspace_bytes, void *stream) {
    const int st = check_shape(n, out, in);
    if (st != Q4_0_OK) return st;
    if (!valid_dtype(x_dtype)) return Q4_0_EINVAL;
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
    const size_t rbytes = (size_t)pairs * 4u;
    if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, experts, wbytes) ||
        overlaps(y, ybytes, route, rbytes))
        return Q4_0_EALIAS;
    const int form = routed_form(n, k, n_experts, out, in, route_kernel);
    if (form < 0) return form;
    const Span spans[4] = {{experts, wbytes}, {x, xbytes}, {route, rbytes}, {y, ybytes}};
    const int wst = check_workspace(workspace, workspace_bytes,
                                    routed_workspace(form, n, k, n_experts, out, in), spans, 4);
    if (wst != Q4_0_OK) return wst;
    const hipStream_t s = (hipStream_t)stream;
    const int f16 = x_dtype == Q4_0_F16;
    return map_hip(form == Q4_0_ROUTE_BY_COLUMN
                       ? q4::launch_gemv_mfma_routed(experts, n_experts, x, f16, route, k, y, n,
                                                     out, in, workspace, s)
                       : q4::launch_gemv_mfma_by_expert(experts, n_experts, x, f16, route, k, y,
                                                        n, out, in, workspace, s));
}

int q4_0_matmul_routed(const void *experts, int64_t n_experts, const void *x, int x_dtype,
                       const int32_t *route, int64_t k, float *y, int64_t n, int64_t out,
                       int64_t in, void *workspace, size_t workspace_bytes, void *stream) {
    return q4_0_matmul_routed_ex(experts, n_experts, x, x_dtype, route, k, y, n, out, in,
                                 Q4_0_ROUTE_AUTO, workspace, workspace_bytes, stream);
}

int q4_0_grouped_workspace_size(const q4_0_linear *linears, int count, int x_dtype,
                                int64_t n, size_t *bytes) {
    if (!bytes) return Q4_0_ENULL;
    GroupPlan gp;
    const int st = plan_group(linears, count, x_dtype, n, &gp);
    if (st != Q4_0_OK) return st;
    *bytes = gp.ws;
    return Q4_0_OK;
}

int q4_0_matmul_grouped(const q4_0_linear *linears, int count, int x_dtype, int64_t n,
                        void *workspace, size_t workspace_bytes, void *stream) {
    GroupPlan gp;
    int st = plan_group(linears, count, x_dtype, n, &gp);
    if (st != Q4_0_OK) return st;
    // every linear is checked, and the workspace against all of them, before
    // anything is enqueued
    Span spans[3 * Q4_0_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        st = check_linear(linears, count, i, x_dtype, n);
        if (st != Q4_0_OK) return st;
        const q4_0_linear &L = linears[i];
        spans[3 * i] = {L.packed, (size_t)q4::Layout(L.out, L.in).total_bytes()};
        spans[3 * i + 1] = {L.x, (size_t)n * (size_t)L.in * (size_t)elem_bytes(x_dtype)};
        spans[3 * i + 2] = {L.y, (size_t)n * (size_t)L.out * 4u};
    }
    st = check_workspace(workspace, workspace_bytes, gp.ws, spans, 3 * count);
    if (st != Q4_0_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    const int x_f16 = x_dtype == Q4_0_F16;
    if (!gp.one_launch) {
        for (int i = 0; i < count; ++i) {
            const q4_0_linear &L = linears[i];
            st = launch_kernel(gp.kernels[i], L.packed, L.x, x_f16, L.y, n, L.out, L.in,
                               workspace, s);
            if (st != Q4_0_OK) return st;
        }
        return Q4_0_OK;
    }
    q4::GemvProblem probs[Q4_0_MAX_GROUP];
    for (int i = 0; i < count; ++i)
        probs[i] = {linears[i].packed, linears[i].x, linears[i].y, linears[i].out,
                    linears[i].in};
    // one launch per slice of up to `lr` rows of every x and y
    const int64_t esize = elem_bytes(x_dtype);
    const int64_t lr = q4::gemv_mfma_launch_rows(probs, count);
    for (int64_t r0 = 0; r0 < n; r0 += lr) {
        const int64_t nr = n - r0 < lr ? n - r0 : lr;
        q4::GemvProblem ps[Q4_0_MAX_GROUP];
        for (int i = 0; i < count; ++i)
            ps[i] = {probs[i].packed, (const uint8_t *)probs[i].x + r0 * probs[i].in * esize,
                     probs[i].y + r0 * probs[i].out, probs[i].out, probs[i].in};
        st = map_hip(q4::launch_gemv_mfma_group(ps, count, nr, x_f16, workspace, s));
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

int q4_0_stream_read(const void *src, int64_t bytes, float *sink, int64_t workgroups,
                     void *stream) {
    if (bytes < 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536)
        return Q4_0_EINVAL;
    if (!sink || (bytes > 0 && !src)) return Q4_0_ENULL;
    if (!aligned(src, 16) || !aligned(sink, 4)) return Q4_0_EALIGN;
    if (overlaps(sink, (size_t)workgroups * 4u, src, (size_t)bytes)) return Q4_0_EALIAS;
    return map_hip(q4::launch_stream_read(src, bytes, sink, workgroups, (hipStream_t)stream));
}

const char *q4_0_strerror(int status) {
    switch (status) {
    case Q4_0_OK: return "success";
    case Q4_0_EINVAL: return "invalid dtype or kernel selector";
    case Q4_0_ESHAPE: return "invalid shape (need n, out >= 1, in >= 32, in % 32 == 0, within limits)";
    case Q4_0_ENULL: return "null pointer argument";
    case Q4_0_EALIGN: return "misaligned pointer (packed and x need 16 bytes, y 4 bytes, workspace 256)";
    case Q4_0_EALIAS: return "an output or the workspace overlaps another buffer of the call";
    case Q4_0_EUNSUPPORTED: return "the requested kernel cannot take this shape";
    case Q4_0_EHIP: return "HIP runtime error at launch";
    case Q4_0_EWORKSPACE: return "workspace missing or smaller than the call needs";
    default: return "unknown status";
    }
}

int q4_0_version(void) { return 20000; }

}  // extern "C"
