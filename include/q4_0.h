/*
 * libq4_0: GGUF Q4_0 block-quantized weight matmul on one AMD MI355X (gfx950).
 *
 *     y[n x out] = x[n x in] . W^T,   W[out x in] in Q4_0 blocks.
 *
 * W is stored the way rembed's matmul interface stores a linear layer's
 * weight (rembed "Architecture", "The pluggable kernel interface"): [out x in]
 * row-major, so each output is the dot product of a weight row with an
 * activation row.  Each row is cut into groups of 32 weights along `in`
 * (goinfer primer ch. 10, "Making Go fast enough": groups of 32, a scale plus
 * small integers two to a byte).  A GGUF Q4_0 block is 18 bytes: the group's
 * scale d as IEEE binary16, little-endian, then 16 code bytes in the
 * split-half order of goinfer ch. 10 "Layout, concretely" (byte i: weight i in
 * the low four bits, weight i+16 in the high four bits).  Weight = d * (q - 8).
 *
 * Conventions for every entry point:
 *  - Pointers to weights, activations, outputs and workspaces are DEVICE
 *    pointers owned by the caller.  The library allocates no memory, never
 *    synchronizes the host with the device, keeps no state between calls
 *    and enqueues its work only on `stream` (a hipStream_t; NULL is the null
 *    stream of the current device).  The current HIP device must be the one
 *    holding the buffers.  Every call may therefore be captured into a HIP
 *    graph, the first call of a process included.
 *  - Workspace: some calls need device scratch memory (partial sums of a K
 *    range split across workgroups; activations converted once into the
 *    matrix-core operand layout; routing tables).  Each such call takes
 *    `workspace` and `workspace_bytes`; the matching *_workspace_size query
 *    (host only, no HIP call) gives the bytes the call needs, 0 when it
 *    needs none (then `workspace` may be NULL).  A workspace must be 256-byte
 *    aligned, overlap no argument of the call, and hold at least the queried
 *    bytes (Q4_0_EWORKSPACE otherwise).  Its contents on entry do not matter
 *    and are undefined afterwards.  Calls whose work may overlap in time
 *    (different streams, graph replays) must use different workspaces;
 *    calls ordered on one stream may share one.  No call needs more than
 *    Q4_0_WORKSPACE_MAX bytes: one buffer of that size serves every call.
 *    The sizes depend on the current device's compute-unit count, which
 *    sets how work is split.
 *  - Arguments are validated on the host before any HIP call; an invalid
 *    call returns a negative Q4_0_E* status and enqueues nothing.  Launch
 *    failures return Q4_0_EHIP.  Errors of work already enqueued (for
 *    example a fault) surface on the stream, as for any HIP kernel.
 *  - No silent fallback: a kernel forced with q4_0_matmul_ex that cannot
 *    take the shape returns Q4_0_EUNSUPPORTED; it never runs another kernel.
 *  - Thread-safe: calls from several host threads may run at once.
 */
#ifndef Q4_0_H
#define Q4_0_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (0 = success). */
#define Q4_0_OK 0
#define Q4_0_EINVAL (-1)       /* unknown dtype or kernel selector            */
#define Q4_0_ESHAPE (-2)       /* n/out/in <= 0, in % 32 != 0, or too large   */
#define Q4_0_ENULL (-3)        /* a required pointer is NULL                  */
#define Q4_0_EALIGN (-4)       /* a pointer is not aligned as required        */
#define Q4_0_EALIAS (-5)       /* an output or the workspace overlaps another
                                  argument                                    */
#define Q4_0_EUNSUPPORTED (-6) /* forced kernel cannot take this shape        */
#define Q4_0_EHIP (-7)         /* the HIP runtime rejected a launch           */
#define Q4_0_EWORKSPACE (-8)   /* workspace missing or smaller than the call
                                  needs                                       */

/* Activation element types. */
#define Q4_0_F32 0             /* float32 x                                   */
#define Q4_0_F16 1             /* IEEE binary16 x                             */

/* Kernel selectors for q4_0_matmul_ex. */
#define Q4_0_KERNEL_AUTO 0      /* what q4_0_matmul runs                      */
#define Q4_0_KERNEL_GEMV_DPP 1  /* small n: VALU dot, x in LDS, DPP/shuffle
                                   reduction; n <= 8                          */
#define Q4_0_KERNEL_GEMV_MFMA 2 /* small n: fp16 MFMA; n <= 8: activations
                                   split into high and low binary16 parts;
                                   9..64: one binary16 part per row; one
                                   launch up to 64 rows (32 for matrices of
                                   4096 tiles or more), row slices above      */
#define Q4_0_KERNEL_GEMM 3      /* prefill: 128 x 128 tiles, weights decoded
                                   to binary16, MFMA                          */

/* Largest sizes accepted (32-bit grid and index limits). */
#define Q4_0_MAX_IN 1048576
#define Q4_0_MAX_OUT 16777216
#define Q4_0_MAX_N 65536
/* Largest workspace any call needs (128 MiB); calls that would need more
 * return Q4_0_EUNSUPPORTED. */
#define Q4_0_WORKSPACE_MAX 134217728
/* Alignment a workspace needs. */
#define Q4_0_WORKSPACE_ALIGN 256

/* Bytes of an [out x in] matrix in GGUF Q4_0 blocks: out * (in/32) * 18.
 * Returns 0 for an invalid shape. */
size_t q4_0_blocks_bytes(int64_t out, int64_t in);

/* Bytes of the repacked matrix.  The repacked matrix is cut into 16-row
 * tiles and each row's blocks into groups of 4, so out is rounded up to a
 * multiple of 16 and in/32 to a multiple of 4 (padding blocks decode to
 * zero):  ceil(out/16)*16 * ceil(in/128)*4 * 18.  Equal to
 * q4_0_blocks_bytes exactly when out % 16 == 0 and in % 128 == 0; larger by
 * at most 15 rows and 3 blocks per row otherwise.  Returns 0 for an invalid
 * shape. */
size_t q4_0_packed_bytes(int64_t out, int64_t in);

/* One-time repack of GGUF Q4_0 blocks into the kernels' layout: goinfer ch. 10
 * "Making Go fast enough" (quantized weights rearranged once so the kernel
 * reads them in order) and "Layout, concretely".  The split-half order inside
 * a block is kept; scales and codes go to two separate streams, each read
 * with wide coalesced loads.  The repacked copy replaces the GGUF one: no
 * second copy is kept alongside it, unlike the opt-in repack that section
 * prices at +80% memory.
 *   blocks : [out][in/32] GGUF blocks, q4_0_blocks_bytes(out,in) bytes,
 *            any alignment.
 *   packed : q4_0_packed_bytes(out,in) bytes, 16-byte aligned, must not
 *            overlap `blocks` (Q4_0_EALIAS).  Fully overwritten.
 * The bytes are moved unchanged: q4_0_unpack restores `blocks` bit for bit,
 * NaN and Inf scales included.  The caller may free `blocks` once the stream
 * has passed this call. */
int q4_0_repack(const void *blocks, void *packed, int64_t out, int64_t in,
                void *stream);

/* Inverse of q4_0_repack: writes the q4_0_blocks_bytes(out,in) GGUF bytes
 * (padding rows and blocks are dropped).  Same alignment and overlap rules. */
int q4_0_unpack(const void *packed, void *blocks, int64_t out, int64_t in,
                void *stream);

/* y = x . W^T with W repacked by q4_0_repack.  The two workloads are the
 * goinfer primer ch. 10 "What the kernels are" pair: the memory-bound decode
 * product (few activation rows, the weights read once for all of them, as in
 * golem's continuous batching, golem README "Several conversations, one
 * pass") and the prefill product (hundreds of rows, compute-bound).
 *   packed : repacked W, 16-byte aligned.
 *   x      : [n x in] row-major, element type x_dtype (Q4_0_F32 or
 *            Q4_0_F16), 16-byte aligned.
 *   y      : [n x out] row-major float32, 4-byte aligned, fully overwritten,
 *            must not overlap `packed` or `x`.
 *   n, out, in : 1 <= n <= Q4_0_MAX_N, 1 <= out <= Q4_0_MAX_OUT,
 *            32 <= in <= Q4_0_MAX_IN, in % 32 == 0.
 *   workspace, workspace_bytes : see the conventions above;
 *            q4_0_matmul_workspace_size with Q4_0_KERNEL_AUTO gives the need.
 * Accuracy, as max |y - y_exact| / sum_k |w x| over outputs: <= 1e-3 on the
 * small-n kernels for n <= 8 (float32 accumulation, 22-bit activations),
 * <= 1e-2 where activations are rounded to binary16: the small-n MFMA kernel
 * above 8 rows and the prefill kernel (which also rounds the weights). */
int q4_0_matmul(const void *packed, const void *x, int x_dtype, float *y,
                int64_t n, int64_t out, int64_t in, void *workspace,
                size_t workspace_bytes, void *stream);

/* q4_0_matmul with the kernel chosen by the caller (tests, benchmarks).
 * Q4_0_KERNEL_AUTO behaves exactly as q4_0_matmul. */
int q4_0_matmul_ex(const void *packed, const void *x, int x_dtype, float *y,
                   int64_t n, int64_t out, int64_t in, int kernel,
                   void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory at all (code under HIP
 * graph capture that may not allocate, tight serving loops, harnesses that
 * forbid hipMalloc): q4_0_matmul with its scratch memory taken from a
 * buffer of Q4_0_STATIC_SCRATCH_BYTES that the library holds in device
 * memory, one per GPU, for the life of the process.  Arguments, results and
 * errors as q4_0_matmul (the same kernels run); Q4_0_EWORKSPACE when the call
 * would need more scratch than that (q4_0_matmul_workspace_size tells).
 * Every call on a GPU shares that GPU's buffer: calls whose work overlaps
 * in time on one GPU (different streams, concurrent graph replays) race and
 * give wrong results; calls ordered on one stream are safe.  Nothing in the
 * buffer needs to start at zero; it keeps the last call's contents. */
#define Q4_0_STATIC_SCRATCH_BYTES 16777216
int q4_0_matmul_static(const void *packed, const void *x, int x_dtype, float *y,
                       int64_t n, int64_t out, int64_t in, void *stream);

/* Workspace bytes of q4_0_matmul_ex with these sizes and kernel (AUTO: of
 * q4_0_matmul) into *bytes.  Host only.  Returns Q4_0_OK, or the status the
 * call itself would return for an invalid shape, dtype or selector, or
 * Q4_0_EUNSUPPORTED. */
int q4_0_matmul_workspace_size(int64_t n, int64_t out, int64_t in, int x_dtype,
                               int kernel, size_t *bytes);

/* One linear of a group: y = x . W^T with the conventions of q4_0_matmul
 * (packed: repacked W, 16-byte aligned; x: [n x in] row-major, 16-byte
 * aligned; y: [n x out] float32, fully overwritten). */
typedef struct q4_0_linear {
    const void *packed;
    const void *x;
    float *y;
    int64_t out, in;
} q4_0_linear;

#define Q4_0_MAX_GROUP 8

/* Several linears that share n and the activation type, e.g. the Q, K and V
 * projections of one input, or the gate and up projections of a feed-forward
 * block.  golem README "Several conversations, one pass": one read of the
 * weights carries every column of the batch; here one launch also carries
 * every weight matrix of the group, so the per-launch cost and the tail of
 * each launch are paid once.
 *   linears : HOST array of `count` descriptors, 1 <= count <= Q4_0_MAX_GROUP;
 *             each is checked as q4_0_matmul checks its arguments.
 *   No y may overlap any x, any packed W or another y of the group
 *   (Q4_0_EALIAS).  The x of different linears may be the same buffer.
 *   workspace, workspace_bytes : q4_0_grouped_workspace_size gives the need.
 * When q4_0_matmul would run the small-n MFMA kernel on every linear
 * (n <= 64 for the usual shapes) the group runs as one launch per 64 rows
 * (32 when a matrix has 4096 tiles or more; above 32 rows the linears must
 * agree), plus the activation pre-pass from 17 rows (from 5 for matrices of
 * 4096 tiles or more) and a reduction launch if a linear splits K; otherwise
 * each linear runs as q4_0_matmul would, in array order, sharing the
 * workspace one after the other.  Every linear is checked before anything is
 * enqueued.  Results equal those of q4_0_matmul on each linear alone. */
int q4_0_matmul_grouped(const q4_0_linear *linears, int count, int x_dtype, int64_t n,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of q4_0_matmul_grouped for this group into *bytes (only
 * the shapes of the descriptors are read).  Host only. */
int q4_0_grouped_workspace_size(const q4_0_linear *linears, int count, int x_dtype,
                                int64_t n, size_t *bytes);

/* Mixture-of-experts product (golem-server README, "On the card": each
 * column is multiplied by the experts its router chose; the column-wise
 * kernels find a column's input through an offset):
 *     y[t*k + j][o] = sum_i W_e[o][i] * x[t][i],   e = route[t*k + j],
 * for every column t < n and slot j < k, on the small-n MFMA kernel, by
 * column or by expert as q4_0_select_route picks (q4_0_matmul_routed_ex).
 *   experts : DEVICE, n_experts repacked [out x in] matrices back to back,
 *             q4_0_packed_bytes(out, in) bytes apart, 16-byte aligned;
 *   x       : DEVICE [n x in] (x_dtype); route : DEVICE int32 [n x k];
 *   y       : DEVICE float32 [n*k x out], overwritten, overlapping neither
 *             x, the experts nor route (Q4_0_EALIAS).
 *   workspace, workspace_bytes : q4_0_routed_workspace_size gives the need.
 * 1 <= n_experts <= Q4_0_MAX_EXPERTS, 1 <= k <= Q4_0_MAX_ROUTED.  The routing
 * stays on the device (no host round trip); an index outside [0, n_experts)
 * reads expert 0 and makes that pair's row NaN.  Q4_0_EUNSUPPORTED when the
 * call would need more than Q4_0_WORKSPACE_MAX bytes of workspace. */
#define Q4_0_MAX_EXPERTS 4096
#define Q4_0_MAX_ROUTED 64
int q4_0_matmul_routed(const void *experts, int64_t n_experts, const void *x, int x_dtype,
                       const int32_t *route, int64_t k, float *y, int64_t n, int64_t out,
                       int64_t in, void *workspace, size_t workspace_bytes, void *stream);

/* The routed product with its form chosen by the caller (golem-server README,
 * "On the card"; by column, each pair reads its own expert's weights; by
 * expert, the columns that share an expert are served by one read of it):
 *   Q4_0_ROUTE_BY_COLUMN : one one-row product per pair, all in one launch;
 *   Q4_0_ROUTE_BY_EXPERT : one workgroup of a pre-pass buckets the pairs
 *       by expert on the device and cuts each bucket into chunks of 8 rows
 *       while the others convert each x row once (binary16 high and low
 *       parts, as q4_0_matmul at n = 8); then each chunk is one 8-row
 *       product with its expert, its rows stored to their pairs' y rows.
 *       Needs n*k <= 4096;
 *   Q4_0_ROUTE_AUTO      : by expert from a measured number of x rows up,
 *       by column below (q4_0_select_route).
 * Both forms give each pair's row to the small-n tolerance of the oracle; a
 * pair's row does not depend on the other pairs.  Arguments and errors as
 * q4_0_matmul_routed, plus Q4_0_EINVAL for an unknown route_kernel and
 * Q4_0_EUNSUPPORTED when the chosen form cannot take the call. */
#define Q4_0_ROUTE_AUTO 0
#define Q4_0_ROUTE_BY_COLUMN 1
#define Q4_0_ROUTE_BY_EXPERT 2
int q4_0_matmul_routed_ex(const void *experts, int64_t n_experts, const void *x, int x_dtype,
                          const int32_t *route, int64_t k, float *y, int64_t n, int64_t out,
                          int64_t in, int route_kernel, void *workspace,
                          size_t workspace_bytes, void *stream);
/* The form Q4_0_ROUTE_AUTO takes for these sizes (a Q4_0_ROUTE_* value), or
 * a negative status (Q4_0_ESHAPE, Q4_0_EINVAL, Q4_0_EUNSUPPORTED). */
int q4_0_select_route(int64_t n, int64_t k, int64_t n_experts, int64_t out, int64_t in);
/* Workspace bytes of q4_0_matmul_routed_ex with these sizes and form into
 * *bytes.  Host only. */
int q4_0_routed_workspace_size(int64_t n, int64_t k, int64_t n_experts, int64_t out,
                               int64_t in, int route_kernel, size_t *bytes);

/* Logit-head product with its epilogue fused: y = x . W^T as in
 * q4_0_matmul (small-n kernel, n <= 64), and for every row t of y its
 * largest value max_val[t] and that value's index max_idx[t] (the smallest
 * index among equal values; NaN never wins; index -1 and a NaN value if no
 * output of the row is a number).  The output head is the largest matrix of
 * a decoder and is read once per pass for every state being scored (golem
 * README, continuous batching: "Several conversations, one pass"); here the
 * greedy pick is taken while the outputs are still on chip, so a caller that
 * only needs the pick can pass y = NULL and no n x out array is written.
 *   y       : [n x out] float32 or NULL.
 *   max_val : n floats, max_idx : n int32, 4-byte aligned, overlapping
 *             nothing else.
 *   workspace, workspace_bytes : q4_0_argmax_workspace_size gives the need
 *             (never 0: the per-workgroup candidates live there).
 * Returns Q4_0_EUNSUPPORTED for shapes the small-n MFMA kernel cannot take
 * (n > 64 among them).  max_val[t] is bit-identical to y[t][max_idx[t]] of
 * the same call. */
int q4_0_matmul_argmax(const void *packed, const void *x, int x_dtype, float *y, int64_t n,
                       int64_t out, int64_t in, float *max_val, int32_t *max_idx,
                       void *workspace, size_t workspace_bytes, void *stream);
/* Workspace bytes of q4_0_matmul_argmax into *bytes.  Host only. */
int q4_0_argmax_workspace_size(int64_t n, int64_t out, int64_t in, int x_dtype, size_t *bytes);

/* W4A8, the step before the product: quantize activations to 8-bit
 * integers, one scale per 32 values of a row (the weights' block size).
 * rembed "Architecture", "int8 quantization" (activations quantized, an
 * integer dot, an offset correction in the epilogue, an exact integer
 * reference); goinfer primer ch. 10 (the quantized dot on 8-bit integer
 * dot-product hardware).  The pages do not give the scale granularity; this
 * library reads it as per 32-value block:
 *     d[t][b] = max_k |x[t][32b + k]| / 127              (float32 division)
 *     q[t][k] = x[t][k] / d[t][b], rounded to nearest, ties to even
 *               (float32 division), or 0 when d is not positive and finite.
 *   x : [n x in] float32 or binary16, 16-byte aligned.
 *   q : [n x in] int8, 16-byte aligned;  d : [n x in/32] float32.
 * q and d are bit-identical to any correctly rounded float32 evaluation of
 * these formulas.  Needs no workspace. */
int q4_0_quantize_x8(const void *x, int x_dtype, int8_t *q, float *d, int64_t n, int64_t in,
                     void *stream);

/* W4A8 product on quantized activations (q, d from q4_0_quantize_x8):
 *     y[t][o] = sum_b dw[o][b] * d[t][b] * sum_{k in b} (qw[o][k] - 8) * q[t][k]
 * with exact integer block sums on the integer matrix cores (the offset 8
 * subtracted as 8 * sum_k q, rembed's colSum correction) and float32 scaling
 * and accumulation: |y - y_exact| <= 1e-4 * sum_b |dw d| sum_k |(qw-8) q|.
 * n <= 64 (one launch per 16 rows).  y: [n x out] float32, overwritten,
 * overlapping neither W, q nor d.  workspace, workspace_bytes:
 * q4_0_w4a8_workspace_size gives the need. */
int q4_0_matmul_w4a8(const void *packed, const int8_t *q, const float *d, float *y, int64_t n,
                     int64_t out, int64_t in, void *workspace, size_t workspace_bytes,
                     void *stream);
/* Workspace bytes of q4_0_matmul_w4a8 into *bytes.  Host only. */
int q4_0_w4a8_workspace_size(int64_t n, int64_t out, int64_t in, size_t *bytes);

/* The kernel q4_0_matmul would run for this call shape (a Q4_0_KERNEL_*
 * value), or a negative status for an invalid shape.  Host only. */
int q4_0_select_kernel(int64_t n, int64_t out, int64_t in, int x_dtype);

/* Whether `kernel` can take this shape: Q4_0_OK, Q4_0_EUNSUPPORTED, or
 * another negative status for an invalid shape or selector.  Host only. */
int q4_0_kernel_supports(int kernel, int64_t n, int64_t out, int64_t in,
                         int x_dtype);

/* Measurement aid for benchmarks, not a product call: benchmarks state the
 * large-n kernel's MFMA utilisation against the published peak and against
 * this loop's measured rate (under a sustained matrix load the part runs
 * below its boost clock).  Enqueues `workgroups` workgroups of four waves, one wave per
 * SIMD, each issuing `iters` x 8 independent v_mfma_f32_32x32x16_f16 back to
 * back, and writes one checksum per thread to sink[workgroups * 256] (device
 * float32, caller-owned).  *flops receives the floating-point operations the
 * launch performs (host pointer); the caller times the launch on `stream`.
 * 1 <= workgroups <= 65536 and 1 <= iters <= 1e6, else Q4_0_EINVAL. */
int q4_0_mfma_loop(float *sink, int64_t workgroups, int64_t iters, int64_t *flops,
                   void *stream);

/* Measurement aid for benchmarks, not a product call: the read rate a plain
 * streaming kernel reaches for a given size, the attainable ceiling beside
 * the published HBM peak for the small-n kernels (which read each weight
 * byte once).  Enqueues `workgroups` workgroups of 256 threads that read
 * the `bytes` bytes at `src` once, 16 bytes per load with non-temporal
 * loads, and write one checksum per workgroup to sink[workgroups] (device
 * float32).  bytes == 0 enqueues the same grid with nothing to read: the
 * cost of one launch.
 *   src : 16-byte aligned (may be NULL when bytes == 0);
 *   0 <= bytes, bytes % 16 == 0; 1 <= workgroups <= 65536, else
 *   Q4_0_EINVAL (Q4_0_ENULL, Q4_0_EALIGN as usual). */
int q4_0_stream_read(const void *src, int64_t bytes, float *sink, int64_t workgroups,
                     void *stream);

/* Static text for a status code. */
const char *q4_0_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int q4_0_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4_0_H */
