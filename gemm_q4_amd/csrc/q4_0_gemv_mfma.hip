// Small-n Q4_0 product on the matrix cores: y[n x out] = x . W^T for up to
// 64 rows per launch, for one linear or for a group of linears that share n
// in one launch.
//
// Why MFMA for a memory-bound product: a vector-ALU dot costs about n + 1.25
// VALU operations per weight, more than the ~3.9 per weight that 70% of HBM
// bandwidth leaves on gfx950 once n reaches 4 or so (golem's card hits the
// same wall past a few columns, golem-server README "On the card").  Here the
// VALU only decodes (about 1.7 operations per weight, independent of n) and
// one v_mfma_f32_16x16x32_f16 per Q4_0 block does all n dot products at once.
//
// Operands of one MFMA (M = 16 activation slots, N = 16 weight rows, K = 32 =
// one Q4_0 block):
//   A: slot m < 8 holds the binary16 high part of activation row m, slot
//      8 + m its low part x - hi (also binary16).  hi + lo carries 22 bits of
//      x.  Before the split each wave scales each activation row of its own K
//      range by a power of two chosen from the row's largest |x| there (no
//      binary16 overflow, no underflow of the low part); the scale is undone
//      exactly on the wave's partial sums.  The wave converts its range of x
//      once, into its own region of LDS, laid out as A fragments (16 bytes per
//      lane and block), and reuses them for every tile it visits.
//   B: exact q - 8 in binary16, decoded straight from the repacked code word
//      the lane loaded (no LDS round trip).
//   D: lane l holds slots 4*(l/16)+i, i = 0..3, of weight row l%16; per block
//      acc += d * D in float32 (d is the row's binary16 scale).
// hi and lo slots of a row are summed with one cross-lane shuffle (xor 32).
// From 9 rows (the band between decode and prefill) each row takes one slot
// holding its scaled binary16 value, without a low part: the precision of the
// prefill kernel, which rounds x to binary16 as well (2^-11 relative).  Above
// 16 rows further A operands hold rows 16..63 (up to four 16-row groups) and
// each decoded B fragment feeds all their products, so the weights are still
// read once.
//
// Work split.  A workgroup owns a run of 16-row tiles of one linear and one
// of its S slices of K; its waves take contiguous runs of `per` <= GPW
// 4-block groups of the slice, every tile of the run.  Each wave first
// requests its range of x, then all of the first tile's code and scale words
// (unconditionally: a wave with fewer than GPW groups repeats a valid
// address, so the memory counter lets every consumer wait for exactly its own
// words), and stages its x while the weights are in flight.  No step before
// the first product waits for another wave.  Each later tile's words are
// requested as the current tile's are consumed.  The waves' per-tile partial
// sums are parked in LDS and summed, in wave order, once per run of up to
// kRedTiles tiles (one workgroup barrier per run, not per tile).  K is split
// (S > 1) only when the slice's A fragments would not fit the LDS budget;
// then each workgroup parks its per-tile sums in a workspace and a second
// small kernel adds the S slices in slice order.  The kernel boundary orders
// the two, so no device-wide fence or atomic is needed (on this multi-die
// part such a fence writes back and invalidates L2).
//
// Groups of linears (golem README "Several conversations, one pass": one
// read of the weights carries every column; here one launch also carries
// several weight matrices, e.g. the Q, K and V projections of one input):
// the workgroups of a launch are dealt to the linears in order, each linear
// with its own plan; the launch's wave count is the largest plan's, and the
// extra waves of a smaller plan have no groups (in the IDLE instance they skip
// the tiles and only join the reductions).
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

// Workgroups a launch aims for, per compute unit of the device.  Each
// workgroup stages (or, from kPrepMinN rows on, loads as prepared fragments)
// the x of its whole K range once and walks a run of tiles with it; from four
// rows on those fragments outweigh one 16-row tile's weights, so short runs
// multiply the traffic.  Measured on MI355X (256 compute units, graph
// replay): up to a few thousand tile-slices about one workgroup per compute
// unit is best (FFN-up 9728 x 2560, n = 1/4/8: 6.0/8.8/10.1 us against
// 6.3/9.9/11.3 us with one tile per workgroup); the 151936-row logit head
// wants about two per compute unit (n = 1/4: 36.0/41.7 us against 36.7/43.7
// us with four and 36.7/42.9 with three: at four rows its prepared instance
// holds 158 VGPRs, three waves per SIMD, so four per compute unit left a
// tail of workgroups that were not resident).
#ifndef Q4_MFMA_WGS_PER_CU
#define Q4_MFMA_WGS_PER_CU 2
#endif
#ifndef Q4_MFMA_WGS_PER_CU_SMALL
#define Q4_MFMA_WGS_PER_CU_SMALL 1
#endif
#ifndef Q4_MFMA_MANY_TILES
#define Q4_MFMA_MANY_TILES 4096
#endif
// LDS for a workgroup's staged A fragments; a K range whose fragments exceed
// it is split.  Measured on MI355X: 96 KB keeps the block's 2560 x 9728 down
// projection (76 groups) in one K slice at n = 2 and in two at n = 4
// (grouped block n = 2/4: 29.0/35.8 us against 30.0/37.2 us with 56 KB);
// 128 or 144 KB change nothing measured (the block as four grouped calls at
// n = 8: 40.4/40.6 us against 40.7 us).
#ifndef Q4_MFMA_LDS_BUDGET
#define Q4_MFMA_LDS_BUDGET (96 * 1024)
#endif
#ifndef Q4_MFMA_GROUPS_PER_WAVE
#define Q4_MFMA_GROUPS_PER_WAVE 5
#endif
constexpr int kMfmaMaxWaves = 8;
constexpr int kMaxRows = (int)kGemvLaunchRows;   // activation rows of one launch
constexpr int kArgmaxRows = 16;                  // rows of one fused greedy-pick launch
// rows <= 8: high and low binary16 part of each row (2n slots); 9..16 rows:
// one binary16 slot per row
template <int NT> constexpr bool split_rows() { return NT <= 8; }
template <int NT> constexpr int row_slots() { return NT <= 8 ? 2 * NT : NT; }
// Kernel instance for a launch of n rows: exact up to 32 rows, then 48 or 64
// rows with the launch's own row count bounding what is read and stored.
constexpr int64_t kernel_rows(int64_t n) { return n <= 32 ? n : (n <= 48 ? 48 : 64); }
static int64_t slots_for(int64_t n) {
    n = kernel_rows(n);
    return n <= 8 ? 2 * n : n;
}
// A group of linears in one launch aims for this many workgroups per compute
// unit over all its linears, each linear's share in proportion to its weight
// bytes (tiles x groups per row, so a workgroup's run takes about as long in
// every linear):
// targets taken per linear would add up to several workgroups per compute
// unit, each walking short runs of tiles and loading its K range of x (at
// eight rows, 80-152 KB of prepared fragments) for each short run.
#ifndef Q4_MFMA_GROUP_WGS_PER_CU
#define Q4_MFMA_GROUP_WGS_PER_CU 1
#endif
// Routed launches aim for this many workgroups per compute unit over all
// their pairs or chunks (measured with 128 experts of 768 x 2048: about 1024
// workgroups in all, 2048-8192 no better).
#ifndef Q4_MFMA_ROUTED_WGS_PER_CU
#define Q4_MFMA_ROUTED_WGS_PER_CU 4
#endif
// workgroups a launch aims for on this device: many tiles, fewer tiles
static int64_t target_wgs() { return (int64_t)device_shape().cus * Q4_MFMA_WGS_PER_CU; }
static int64_t target_wgs_small() {
    return (int64_t)device_shape().cus * Q4_MFMA_WGS_PER_CU_SMALL;
}
constexpr int64_t kMfmaManyTiles = Q4_MFMA_MANY_TILES;
constexpr int64_t kMfmaLdsBudget = Q4_MFMA_LDS_BUDGET;   // A fragments per workgroup
// x items (8 values each) a lane holds while it stages: caps groups per wave
// x rows (the 16-row instance staging five groups holds 221 VGPRs, no spills)
#ifndef Q4_MAX_STAGE_ITEMS
#define Q4_MAX_STAGE_ITEMS 20
#endif
constexpr int kMaxStageItems = Q4_MAX_STAGE_ITEMS;
// Activation rows from which x is converted once per launch by a pre-pass
// (xprep_kernel) instead of by every workgroup.  Measured on MI355X (graph
// replay, workgroups walking runs of tiles): FFN-up 9728 x 2560 at n = 4/5
// takes 8.0/8.9 us with per-workgroup conversion against 8.7/9.1 us with the
// pre-pass, and at n = 6/8 10.5/10.8 us against 10.2/10.4 us.  The block of
// seven linears in one grouped call (its workgroups shared out over the
// group: long runs of tiles, so each workgroup converts once for many
// tiles) at n = 6/8 takes 24.1/24.6 us converting per workgroup against
// 25.2/26.7 us with the pre-pass.  The 151936-row head at n = 4, two
// workgroups per compute unit: 40.8 us converting per workgroup against 41.0
// us with the pre-pass, and 45.2 against 46.7 us with the fused greedy pick.
// With the staging that gives each lane one row and twenty staged items per
// lane: FFN-up n = 12/16 11.18/11.34 us converting per workgroup against
// 11.81/11.98 us with the pre-pass, the block as four grouped calls at
// n = 16 49.2 against 51.7 us, in one grouped call at n = 12 26.0 against
// 29.2 us; the head at n = 8 converting per workgroup 60.7 against 47.8 us.
// So the pre-pass from 17 rows (where a second 16-row A group starts, whose
// fragments a wave keeps in registers), and from 5 rows for matrices of at
// least kMfmaManyTiles tiles.
#ifndef Q4_MFMA_PREP_MIN_N
#define Q4_MFMA_PREP_MIN_N 17
#endif
#ifndef Q4_MFMA_PREP_MIN_N_LARGE
#define Q4_MFMA_PREP_MIN_N_LARGE 5
#endif
constexpr int kPrepMinN = Q4_MFMA_PREP_MIN_N;
constexpr int kPrepMinNLarge = Q4_MFMA_PREP_MIN_N_LARGE;
// groups per wave when the A fragments of its range live in registers: 5 with
// one 16-row A group, 4 with two, 2 with three or four
constexpr int kPrepMaxGroups = 5;
constexpr int kPrepMaxGroups2 = 4;    // two A groups (17..32 rows)
constexpr int kPrepMaxGroups4 = 2;    // three or four A groups (33..64 rows)
constexpr int prep_groups(int64_t rows) {
    return rows > 32 ? kPrepMaxGroups4 : (rows > 16 ? kPrepMaxGroups2 : kPrepMaxGroups);
}
template <int NT> constexpr int prep_max_groups() { return prep_groups(NT); }
// prepared fragments: per-row inverse scales (float) in the first 256 bytes
constexpr int kFragHeader = 256;
// tiles whose per-wave partial sums are parked before a workgroup reduction
// (16 KB of LDS whatever n is)
template <int NT> constexpr int red_tiles() { return NT > 32 ? 1 : (32 / NT < 2 ? 2 : 32 / NT); }
// Prepared launches above 16 rows use no dynamic LDS, and their register use
// (210-246 VGPRs) already leaves one workgroup per compute unit, so their
// parked sums may take 96 KB: 3 tiles at 64 rows, 6 at 32 rows, instead of 1
// and 2.  Measured on MI355X (graph replay): FFN-up 9728 x 2560 at n = 32/48
// 13.7/21.6 us against 13.9/22.4 us, the 151936-row head at 32 rows 88.0
// against 91.3 us, the block as four grouped calls at n = 64 101.4 against
// 104.9 us; 64 KB gave about half of that.
constexpr int kPrepRedBytes = 96 * 1024;
template <int NT, bool PREP> constexpr int red_tiles_for() {
    return PREP && NT > 16 ? (kPrepRedBytes / (kMfmaMaxWaves * NT * 64) < 1
                                  ? 1
                                  : kPrepRedBytes / (kMfmaMaxWaves * NT * 64))
                           : red_tiles<NT>();
}
// groups per wave a kernel instance holds in registers
constexpr int kGpwSet[] = {1, 2, 4, 5, 8, 10, 16};

// Rows the x staging lays a wave's lanes over: the power of two >= n.
constexpr int stage_rows(int64_t n) { return n <= 1 ? 1 : (n <= 2 ? 2 : (n <= 4 ? 4 : (n <= 8 ? 8 : 16))); }

// The value of lane l ^ 1 (resp. l ^ 2) within each quad of lanes (DPP
// quad_perm, no LDS).
__device__ __forceinline__ float quad_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                              0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E,
                                                              0xF, 0xF, true));
}

// 2^e with e clamped to the float32 normal range.
__device__ __forceinline__ float pow2f(int e) {
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

template <typename XT> __device__ __forceinline__ float4 load_x4(const XT *p);
template <> __device__ __forceinline__ float4 load_x4<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
template <> __device__ __forceinline__ float4 load_x4<_Float16>(const _Float16 *p) {
    const u2_t a = *reinterpret_cast<const u2_t *>(p);
    const h2_t a0 = as_h2(a[0]), a1 = as_h2(a[1]);
    return float4{(float)a0.x, (float)a0.y, (float)a1.x, (float)a1.y};
}

// One linear of a launch and its plan, computed on the host (the device
// divides once per workgroup, to find its slice).
struct GemvLinear {
    const uint8_t *packed;
    const void *x;
    float *y;
    float *part;         // per-slice partial sums when K is split, else null
    const uint8_t *frag; // x converted by xprep_kernel (prepared launches)
    uint2 *amax;         // per-workgroup (max, index) of each row of y, or null
    int64_t code_base;   // byte offset of the code stream in `packed`
    int out, in;
    int g4, tiles;       // groups per padded row, 16-row tiles
    int gps;             // groups per K slice
    int per;             // groups per wave (<= GPW)
    int tpw;             // tiles per workgroup
    int gx;              // workgroups along the tiles (per slice)
    int wg0;             // first workgroup of this linear in the launch
};

// A routed launch (mixture of experts, by column): lin[0] describes the
// geometry of every expert; pair p = column * k + slot computes row p of y
// from x row p / k and the expert route[p] of a stack of experts.
//
// By expert instead (chunk_expert set): the pairs routed to one expert are
// bucketed into chunks of kChunkRows rows (route_plan), each chunk is
// one kChunkRows-row product with its expert, and wpp workgroups serve each
// chunk; row i of a chunk reads the prepared fragments of x row
// slot_pair[chunk * kChunkRows + i] / k and lands in y row slot_pair[...].
constexpr int kChunkRows = 8;
struct GemvRoute {
    const int32_t *route; // device, one expert index per pair; null: not routed
    const int32_t *chunk_expert; // by expert: expert of each chunk (E: invalid, -1: unused)
    const int32_t *slot_pair;    // by expert: pair of each chunk row (-1: padding)
    int64_t expert_bytes; // bytes from one expert's packed matrix to the next
    int64_t x_row_bytes;  // bytes from one x row to the next
    int64_t part_pair;    // floats of partial sums per pair or chunk (K split), else 0
    int64_t frag_chunk;   // by expert: bytes of one 8-row region of prepared x fragments
    int n_experts;
    int k;                // pairs per x row
    int wpp;              // workgroups per pair or chunk
    int x_rows;           // by expert: rows of x (host side, sizes the pre-pass)
};

struct GemvArgs {
    GemvLinear lin[kMaxGroupLinears];
    int nlin;
    int nrows;            // activation rows of the launch (<= the instance's NT)
    GemvRoute rt;
};

struct MfmaPlan {
    int waves;        // waves the linear uses
    int gpw;          // register capacity per wave (template bound), >= per
    int per;          // groups per wave
    int64_t gps;      // groups per K slice
    int64_t slices;   // S: workgroups along K
    int64_t tpw;      // tiles per workgroup
    int64_t gx;       // workgroups along the tiles
    int64_t lds;      // A-fragment bytes of one workgroup
};

// Scaled binary16 high and low parts of 8 activations, as two A fragments in
// the slot order of decode_word_pairs: k = {0, 2, 16, 18, 1, 3, 17, 19} +
// 4g of a block, from v[] = values at k = 4g + {0, 1, 2, 3, 16, 17, 18, 19}.
__device__ __forceinline__ void split_fragment(const float v[8], float sc, h8_t &fh, h8_t &fl) {
    _Float16 hi[8], lo[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float sv = v[k] * sc;
        hi[k] = (_Float16)sv;
        lo[k] = (_Float16)(sv - (float)hi[k]);
    }
    fh = h8_t{hi[0], hi[2], hi[4], hi[6], hi[1], hi[3], hi[5], hi[7]};
    fl = h8_t{lo[0], lo[2], lo[4], lo[6], lo[1], lo[3], lo[5], lo[7]};
}

// Power-of-two scale that puts a row's largest |x| in [2^14, 2^15) (1 for a
// zero or non-finite maximum), and its exact inverse.
__device__ __forceinline__ float row_scale(float m) {
    if (m > 0.0f && m <= 3.0e38f) {
        const int e = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
        return pow2f(14 - e);
    }
    return 1.0f;
}
__device__ __forceinline__ float inverse_pow2(float sc) {
    return pow2f(127 - (int)(__builtin_bit_cast(uint32_t, sc) >> 23));
}

// Running maximum of a row of y with its index: a larger value wins, an equal
// value with a smaller index wins, a NaN never wins.
__device__ __forceinline__ void amax_update(float v, int i, float &bv, int &bi) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// Workgroup-wide (max, index) of each of NT rows from every thread's
// candidates; thread t < NT stores row t's pair at out[t] (value bits, index).
// Called by every thread of the workgroup.
template <int NT>
__device__ void amax_workgroup(float (&bv)[NT], int (&bi)[NT], uint2 *out) {
    __shared__ uint2 wb[kMfmaMaxWaves][NT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float v = bv[t];
        int i = bi[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(v, off);
            const int oi = __shfl_xor(i, off);
            amax_update(ov, oi, v, i);
        }
        if (lane == 0) wb[wave][t] = uint2{__builtin_bit_cast(uint32_t, v), (uint32_t)i};
    }
    __syncthreads();
    if ((int)threadIdx.x < NT) {
        const int t = threadIdx.x;
        float v = -__builtin_huge_valf();
        int i = 0x7fffffff;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w)
            amax_update(__builtin_bit_cast(float, wb[w][t].x), (int)wb[w][t].y, v, i);
        out[t] = uint2{__builtin_bit_cast(uint32_t, v), (uint32_t)i};
    }
}

// Pre-pass of a prepared launch: converts x [NT x in] once into the A
// fragments every workgroup would otherwise build for itself.  Workgroup t
// converts row t: item (block b, quarter g) holds the 8 values k = 32b + 4g +
// {0..3, 16..19}; each thread loads its items (kPrepItems of them in
// registers, more in further passes that load again), the workgroup finds
// the row's largest |x|, and each item is written as slot j in [0, S)
// (S = 2*NT for NT <= 8: j < NT high part of row j, j >= NT low part of row
// j - NT; S = NT above 8 rows: row j) and quarter g, 16 bytes at
// kFragHeader + ((b * S + j) * 4 + g) * 16.  Blocks past in
// (up to the padded group) are zeros.  Float at byte 4t: the inverse of row
// t's scale.  One memory round trip for rows up to 512 * kPrepItems / 4
// blocks.
constexpr int kPrepThreads = 512;
constexpr int kPrepItems = 4;
template <typename XT>
__device__ __forceinline__ void load_item(const XT *row, int in, int it, float v[8]) {
    const int b = it >> 2, gq = it & 3;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    if (b * 32 < in) {
        const XT *p = row + 32 * b + 4 * gq;
        const float4 u = load_x4<XT>(p), w = load_x4<XT>(p + 16);
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
        v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
    }
}
//
// In regions (region_bytes set, by-expert routing): workgroup w converts x
// row w (zeros past x_rows) as row w % 8 of its own 8-row region of
// fragments, region w / 8, region_bytes apart.
struct XRegions {
    int64_t region_bytes;
    int x_rows;
};
template <int NT, typename XT>
__device__ __forceinline__ void xprep_row(const XT *__restrict__ x, int in, int nbpad,
                                          uint8_t *__restrict__ frag, const XRegions reg,
                                          int t) {
    __shared__ float wmax[kPrepThreads / 64];
    const XT *row = x + (int64_t)t * in;
    if (reg.region_bytes) {
        if (t >= reg.x_rows) {                                // padding: a zero row
            row = x;
            in = 0;
        }
        frag += (int64_t)(t / kChunkRows) * reg.region_bytes;
        t %= kChunkRows;
    }
    const int items = nbpad * 4;
    float v[kPrepItems][8];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kPrepItems; ++i) {
        const int it = threadIdx.x + i * kPrepThreads;
        load_item(row, it < items ? in : 0, it, v[i]);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[i][k]));
    }
    for (int it = threadIdx.x + kPrepItems * kPrepThreads; it < items; it += kPrepThreads) {
        float w[8];
        load_item(row, in, it, w);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(w[k]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    m = wmax[0];
#pragma unroll
    for (int w = 1; w < kPrepThreads / 64; ++w) m = fmaxf(m, wmax[w]);
    const float sc = row_scale(m);
    if (threadIdx.x == 0) reinterpret_cast<float *>(frag)[t] = inverse_pow2(sc);
    uint8_t *f = frag + kFragHeader;
    constexpr int kS = row_slots<NT>();
    auto store = [&](int it, const float w[8]) {
        const int b = it >> 2, gq = it & 3;
        h8_t fh, fl;
        split_fragment(w, sc, fh, fl);
        *reinterpret_cast<h8_t *>(f + ((b * kS + t) * 4 + gq) * 16) = fh;
        if constexpr (split_rows<NT>())
            *reinterpret_cast<h8_t *>(f + ((b * kS + NT + t) * 4 + gq) * 16) = fl;
    };
#pragma unroll
    for (int i = 0; i < kPrepItems; ++i) {
        const int it = threadIdx.x + i * kPrepThreads;
        if (it < items) store(it, v[i]);
    }
    for (int it = threadIdx.x + kPrepItems * kPrepThreads; it < items; it += kPrepThreads) {
        float w[8];
        load_item(row, in, it, w);
        store(it, w);
    }
}

// The pre-pass of a launch: every distinct x of its linears, one workgroup
// per (x, row), in one launch (a group of linears with different inputs,
// e.g. every projection of a decoder block, needs one pre-pass launch, not
// one per input).
struct PrepSet {
    const void *x[kMaxGroupLinears];
    uint8_t *frag[kMaxGroupLinears];
    int in[kMaxGroupLinears];
    int nbpad[kMaxGroupLinears];
    int count;
    int rows;                 // rows of each x (workgroups per x)
};
template <int NT, typename XT>
__global__ __launch_bounds__(kPrepThreads) void xprep_kernel(const PrepSet set) {
    const int e = (int)blockIdx.x / set.rows, t = (int)blockIdx.x - e * set.rows;
    xprep_row<NT, XT>((const XT *)set.x[e], set.in[e], set.nbpad[e], set.frag[e], XRegions{},
                      t);
}

// Routed by expert: the plan.  One workgroup (of kPlanThreads) buckets the pairs p = t*k + j by
// expert (an index outside [0, E) goes to bucket E), cuts each bucket into
// chunks of kChunkRows rows and writes chunk_expert[c] (the bucket of chunk
// c, -1 past the used chunks) and slot_pair[c * kChunkRows + i] (the pair in
// row i of chunk c, -1 for padding).  A pair's place inside its bucket comes
// from an LDS atomic and may change from call to call; the y row of every
// pair does not, since the rows of a chunk's product are independent.
constexpr int kPlanThreads = kPrepThreads;   // the plan runs as workgroup 0 of the pre-pass
constexpr int kPlanMaxPairs = 4096;
constexpr int kPlanMaxBuckets = 4097;    // experts + the invalid bucket
__device__ __forceinline__ void route_plan(const int32_t *__restrict__ route, int pairs,
                                           int n_experts, int max_chunks,
                                           int32_t *__restrict__ chunk_expert,
                                           int32_t *__restrict__ slot_pair) {
    __shared__ int cnt[kPlanMaxBuckets];   // pairs per bucket, then first chunk of the bucket
    __shared__ int bkt[kPlanMaxPairs];
    __shared__ int rnk[kPlanMaxPairs];
    __shared__ int scan[kPlanThreads];
    const int tid = threadIdx.x;
    const int nb = n_experts + 1;
    for (int i = tid; i < nb; i += kPlanThreads) cnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < pairs; p += kPlanThreads) {
        int e = route[p];
        if (e < 0 || e >= n_experts) e = n_experts;
        bkt[p] = e;
        rnk[p] = atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // chunks per bucket; exclusive scan over contiguous runs of buckets
    const int seg = (nb + kPlanThreads - 1) / kPlanThreads;
    const int s0 = tid * seg < nb ? tid * seg : nb;
    const int s1 = s0 + seg < nb ? s0 + seg : nb;
    int mine = 0;
    for (int i = s0; i < s1; ++i) mine += (cnt[i] + kChunkRows - 1) / kChunkRows;
    scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const int used = scan[kPlanThreads - 1];
    int base = scan[tid] - mine;
    for (int i = s0; i < s1; ++i) {
        const int c = cnt[i], nc = (c + kChunkRows - 1) / kChunkRows;
        for (int q = 0; q < nc; ++q) chunk_expert[base + q] = i;
        for (int q = c; q < nc * kChunkRows; ++q) slot_pair[(int64_t)base * kChunkRows + q] = -1;
        cnt[i] = base;
        base += nc;
    }
    __syncthreads();
    for (int p = tid; p < pairs; p += kPlanThreads)
        slot_pair[(int64_t)cnt[bkt[p]] * kChunkRows + rnk[p]] = p;
    for (int c = used + tid; c < max_chunks; c += kPlanThreads) {
        chunk_expert[c] = -1;
        for (int q = 0; q < kChunkRows; ++q) slot_pair[(int64_t)c * kChunkRows + q] = -1;
    }
}

// The by-expert pre-pass: workgroup 0 makes the plan, workgroup 1 + w
// converts x row w into its region (the two do not depend on each other).
template <int NT, typename XT>
__global__ __launch_bounds__(kPrepThreads) void route_prep_kernel(
    const int32_t *__restrict__ route, int pairs, int n_experts, int max_chunks,
    int32_t *__restrict__ chunk_expert, int32_t *__restrict__ slot_pair,
    const XT *__restrict__ x, int in, int nbpad, uint8_t *__restrict__ frag,
    const XRegions reg) {
    if (blockIdx.x == 0)
        route_plan(route, pairs, n_experts, max_chunks, chunk_expert, slot_pair);
    else
        xprep_row<NT, XT>(x, in, nbpad, frag, reg, (int)blockIdx.x - 1);
}

// A-fragment store of one wave (unprepared launches): for block bl of the
// wave's range, slot j and quarter g as in xprep_kernel, 16 bytes at
// ((bl * 2*NT + j) * 4 + g) * 16 of the wave's LDS region.  A prepared launch
// loads each lane's own fragments of its range straight into registers.
template <int NT, typename XT, int GPW, bool PREP, bool IDLE>
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void gemv_mfma_kernel(const GemvArgs args) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int kRedTiles = red_tiles_for<NT, PREP>();
    __shared__ float red[kRedTiles][kMfmaMaxWaves][NT][16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;

    // ---- which linear, slice and tiles ---------------------------------------
    int li = 0;
    for (int k = 1; k < args.nlin; ++k)
        if ((int)blockIdx.x >= args.lin[k].wg0) li = k;
    GemvLinear a = args.lin[li];
    int local = (int)blockIdx.x - a.wg0;
    // routed launch: this pair's expert, x row, y row and partial sums; an
    // expert index outside the stack reads expert 0 and stores NaN
    bool bad_route = false;
    const int32_t *yslots = nullptr;      // by expert: this chunk's y rows
    if (args.rt.chunk_expert) {
        const int c = (int)blockIdx.x / args.rt.wpp;
        local = (int)blockIdx.x - c * args.rt.wpp;
        int e = __builtin_amdgcn_readfirstlane(args.rt.chunk_expert[c]);
        if (e < 0) return;                // unused chunk: the whole workgroup, before any barrier
        bad_route = e >= args.rt.n_experts;
        if (bad_route) e = 0;
        a.packed += (int64_t)e * args.rt.expert_bytes;
        if (a.part) a.part += (int64_t)c * args.rt.part_pair;
        yslots = args.rt.slot_pair + (int64_t)c * kChunkRows;
    } else if (args.rt.route) {
        const int pair = (int)blockIdx.x / args.rt.wpp;
        local = (int)blockIdx.x - pair * args.rt.wpp;
        int e = __builtin_amdgcn_readfirstlane(args.rt.route[pair]);
        bad_route = e < 0 || e >= args.rt.n_experts;
        if (bad_route) e = 0;
        a.packed += (int64_t)e * args.rt.expert_bytes;
        a.x = (const uint8_t *)a.x + (int64_t)(pair / args.rt.k) * args.rt.x_row_bytes;
        a.y += (int64_t)pair * a.out;
        if (a.part) a.part += (int64_t)pair * args.rt.part_pair;
    }
    const int sy = local / a.gx;                              // K slice
    const int cx = local - sy * a.gx;
    const int gs0 = sy * a.gps;                               // first group of the slice
    const int gsn = a.g4 - gs0 < a.gps ? a.g4 - gs0 : a.gps;  // groups in the slice
    // this wave's groups of the slice: [q0, q0 + ng)
    const int q0 = wave * a.per;
    const int ng = gsn - q0 < 0 ? 0 : (gsn - q0 < a.per ? gsn - q0 : a.per);
    // IDLE instance (a group of linears whose launch has more waves than some
    // linear's plan): waves without groups walk the tiles without requests
    // or products and only join the reductions, whose sums stop at the last
    // wave with groups (the terms left out are exact zeros).  Other launches
    // keep the branch-free loop.
    const int nact = IDLE ? (gsn + a.per - 1) / a.per : nwaves;
    const bool idle = IDLE && ng == 0;
    const int tb = cx * a.tpw;                                // < tiles by the plan
    const int te = tb + a.tpw < a.tiles ? tb + a.tpw : a.tiles;
    const XT *__restrict__ x = (const XT *)a.x;
    const bool split = a.part != nullptr;
    // running (max, index) of each row of y over this thread's outputs (the
    // fused greedy pick runs launches of at most kArgmaxRows rows)
    constexpr int kAm = NT <= kArgmaxRows ? NT : 1;
    float bv[kAm];
    int bi[kAm];
#pragma unroll
    for (int t = 0; t < kAm; ++t) {
        bv[t] = -__builtin_huge_valf();
        bi[t] = 0x7fffffff;
    }

    // Lane's A slot r.  One row: high part in slot 0, low part in slot 8.
    // 2..8 rows (paired): row t's high and low parts in adjacent slots
    // 4(t / kRpg) + 2(t % kRpg) + {0, 1}, so both of its D values sit in one
    // lane's registers (kRpg rows per lane group: 1 up to 4 rows, else 2).
    // Above 8 rows, row r.  Lanes of unused slots read slot 0's fragment: a
    // D row depends only on its own A row, and the rows of unused slots are
    // never read, so their contents do not matter (they stay finite).
    constexpr bool kSplit = split_rows<NT>();
    constexpr bool kPair = kSplit && NT >= 2;
    constexpr int kRpg = NT <= 4 ? 1 : 2;
    int jslot;
    if constexpr (kPair) {
        const int u = (r & 3) >> 1, t = (r >> 2) * kRpg + u;
        jslot = u < kRpg && t < NT ? ((r & 1) ? NT + t : t) : 0;
    } else {
        jslot = r < NT ? r : ((kSplit && r >= 8 && r < 8 + NT) ? NT + (r - 8) : 0);
    }
    // above 16 rows further A groups hold rows 16 j + r, j = 1 .. kRG - 1
    // (prepared x only); each decoded weight fragment then feeds kRG products
    constexpr int kRG = (NT + 15) / 16;
    constexpr int kXG = kRG > 1 ? kRG - 1 : 1;               // array extent of the extra groups
    static_assert(kRG == 1 || PREP, "above 16 rows x is prepared");
    int jslot_x[kXG];
#pragma unroll
    for (int j = 0; j < kXG; ++j) jslot_x[j] = 16 * (j + 1) + r < NT ? 16 * (j + 1) + r : 0;
    constexpr int kBlockFrag = row_slots<NT>() * 64;          // fragment bytes per block
    const int gw = ng > 0 ? gs0 + q0 : gs0;                   // first group of the wave

    // ---- prepared launch: request this lane's fragments ------------------------
    h8_t afr[PREP ? GPW : 1][4];
    h8_t afr_x[kXG][kRG > 1 ? GPW : 1][4];
    if constexpr (PREP) {
        const uint8_t *fb = a.frag + kFragHeader + (jslot * 4 + g) * 16;
        if (yslots) {
            // by expert (8 rows, split): slot j holds the high (j < 8) or low
            // part of chunk row j % 8, whose x row has its own region
            const int pr = yslots[jslot & 7];
            const int xr = pr < 0 ? 0 : pr / args.rt.k;       // padding: row 0, never stored
            fb = a.frag + (int64_t)(xr / kChunkRows) * args.rt.frag_chunk + kFragHeader +
                 (((jslot & 8) + xr % kChunkRows) * 4 + g) * 16;
        }
#pragma unroll
        for (int q = 0; q < GPW; ++q)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int64_t b = (int64_t)(gw + (q < ng ? q : 0)) * 4 + s4;
                afr[q][s4] = *reinterpret_cast<const h8_t *>(fb + b * kBlockFrag);
                if constexpr (kRG > 1) {
#pragma unroll
                    for (int j = 0; j < kRG - 1; ++j)
                        afr_x[j][q][s4] = *reinterpret_cast<const h8_t *>(
                            a.frag + kFragHeader + (jslot_x[j] * 4 + g) * 16 + b * kBlockFrag);
                }
            }
    }

    // ---- otherwise request this wave's range of x -----------------------------
    // item = (block bl, row t, quarter gq): the 8 values k = 32bl + 4gq +
    // {0..3} and 32bl + 16 + 4gq + {0..3} of the wave's range.  The rows are
    // laid over kNTp, the power of two >= NT, so a lane's row t = (lane / 4)
    // mod kNTp is the same for all its items (items of rows >= NT are empty).
    constexpr int kNTp = stage_rows(NT);
    constexpr int kItems = PREP ? 1 : (GPW * 16 * kNTp + 63) / 64;   // per lane
    static_assert(kItems <= kMaxStageItems, "x staging registers");
    const int kw0 = (gs0 + q0) * 128;                         // first k of the range
    const int kwn = ng == 0 ? 0 : (a.in - kw0 < ng * 128 ? a.in - kw0 : ng * 128);
    const int items = ng * 16 * kNTp;
    const int trow = (lane >> 2) & (kNTp - 1);                // this lane's row
    float xv[kItems][8];
#pragma unroll
    for (int ii = 0; ii < kItems; ++ii) {
        const int it = lane + ii * 64;
        const int gq = it & 3;
        const int t = trow;
        const int bl = (it >> 2) / kNTp;
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[ii][k] = 0.0f;
        if (!PREP && t < NT && it < items && bl * 32 < kwn) {
            const XT *p = x + (int64_t)t * a.in + kw0 + 32 * bl + 4 * gq;
            const float4 u = load_x4<XT>(p), v = load_x4<XT>(p + 16);
            xv[ii][0] = u.x; xv[ii][1] = u.y; xv[ii][2] = u.z; xv[ii][3] = u.w;
            xv[ii][4] = v.x; xv[ii][5] = v.y; xv[ii][6] = v.z; xv[ii][7] = v.w;
        }
    }

    // ---- request the first tile's code and scale words --------------------
    // Group q of the wave is slice group q0 + q; a wave with fewer than GPW
    // groups (or none) repeats a valid address of its slice.
    const uint8_t *cbase = a.packed + a.code_base + (int64_t)gw * kGroupCodeBytes + lane * 16;
    const uint8_t *sbase = a.packed + (int64_t)gw * kGroupScaleBytes + r * 8;
    u4_t cw[GPW];
    u2_t sw[GPW];
    auto load_group = [&](int t, int q) {
        const int64_t j = (int64_t)t * a.g4 + (q < ng ? q : 0);
        // read once per call: non-temporal, so the stream does not evict x
        // and the other workgroups' lines from L2
        cw[q] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(cbase + j * kGroupCodeBytes));
        sw[q] = __builtin_nontemporal_load(reinterpret_cast<const u2_t *>(sbase + j * kGroupScaleBytes));
    };
#pragma unroll
    for (int q = 0; q < GPW; ++q) load_group(tb, q);
    // keep the x reduction below the weight requests
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage the wave's x as A fragments -----------------------------------
    // Each row's max |x| over the wave's range: the max over the lane's own
    // items, then over the lanes of its row (those differing in the quarter
    // bits and in the bits above the row's; no LDS for the quarter bits),
    // then each lane scales its items, splits them into high and low binary16
    // parts and writes them as fragments into the wave's own LDS region.
    float scale_l = 1.0f;                                     // this lane's row's scale
    uint8_t *frag = smem + wave * (a.per * 4 * kBlockFrag);
    if constexpr (!PREP) {
    float m = 0.0f;
#pragma unroll
    for (int ii = 0; ii < kItems; ++ii)
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(xv[ii][k]));
    m = fmaxf(m, quad_xor1(m));
    m = fmaxf(m, quad_xor2(m));
#pragma unroll
    for (int off = 4 * kNTp; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    scale_l = row_scale(m);
#pragma unroll
    for (int ii = 0; ii < kItems; ++ii) {
        const int it = lane + ii * 64;
        if (trow < NT && it < items) {
            const int gq = it & 3;
            const int t = trow;
            const int bl = (it >> 2) / kNTp;
            h8_t fh, fl;
            split_fragment(xv[ii], scale_l, fh, fl);
            constexpr int kS = row_slots<NT>();
            *reinterpret_cast<h8_t *>(frag + ((bl * kS + t) * 4 + gq) * 16) = fh;
            if constexpr (kSplit)
                *reinterpret_cast<h8_t *>(frag + ((bl * kS + NT + t) * 4 + gq) * 16) = fl;
        }
    }
    // the fragments are read back by other lanes of this wave only: LDS
    // operations of one wave complete in order, so a wave-level fence keeps
    // the compiler from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const uint8_t *afrag = frag + (jslot * 4 + g) * 16;
    // D slots a lane can hold live: 4g+i for i < kLive
    constexpr int kLive = kPair ? 2 * kRpg : (NT < 4 ? NT : 4);
    // inverse scale of the row behind D slot 4g+i
    float inv[kLive], inv_x[kXG][kLive];
#pragma unroll
    for (int i = 0; i < kLive; ++i) {
        const int row = kPair ? g * kRpg + (i >> 1) : (kSplit ? ((4 * g + i) & 7) : 4 * g + i);
#pragma unroll
        for (int j = 0; j < kXG; ++j) inv_x[j][i] = 1.0f;
        if constexpr (PREP) {
            inv[i] = row < NT ? reinterpret_cast<const float *>(a.frag)[row] : 1.0f;
            if (yslots && row < NT) {
                const int pr = yslots[row];
                const int xr = pr < 0 ? 0 : pr / args.rt.k;
                inv[i] = reinterpret_cast<const float *>(
                    a.frag + (int64_t)(xr / kChunkRows) * args.rt.frag_chunk)[xr % kChunkRows];
            }
            if constexpr (kRG > 1) {
#pragma unroll
                for (int j = 0; j < kRG - 1; ++j) {
                    const int rj = 16 * (j + 1) + row;
                    inv_x[j][i] = rj < NT ? reinterpret_cast<const float *>(a.frag)[rj] : 1.0f;
                }
            }
        } else {
            // the scale of D slot 4g+i's row, from a lane of that row (with
            // one row every lane holds it)
            const float sc = kNTp == 1 ? scale_l : __shfl(scale_l, 4 * (row < NT ? row : 0));
            inv[i] = inverse_pow2(sc);
        }
    }
    const Magic mg = pinned_magic();

    // One tile: per group, four independent products (one per block), then
    // acc += d * D on the live slots.  With `next` set, group q's words of
    // tile t + 1 are requested into the same registers as soon as group q of
    // tile t has consumed them.  The wave's sums are parked in red[slot].
    auto tile = [&](int t, int slot, bool next) {
        float acc[kLive], acc_x[kXG][kLive];
#pragma unroll
        for (int k = 0; k < kLive; ++k) {
            acc[k] = 0.0f;
#pragma unroll
            for (int j = 0; j < kXG; ++j) acc_x[j][k] = 0.0f;
        }
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (q < ng) {
                const uint8_t *ag = afrag + q * 4 * kBlockFrag;
                f4_t dd[4], dd_x[kXG][4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    h8_t av;
                    if constexpr (PREP)
                        av = afr[q][s];
                    else
                        av = *reinterpret_cast<const h8_t *>(ag + s * kBlockFrag);
                    uint32_t qd[4];
                    decode_word_pairs(cw[q][s], mg, qd);
                    const h8_t bw = pack_h8(qd);
                    const f4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
                    dd[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bw, z, 0, 0, 0);
                    if constexpr (kRG > 1) {
#pragma unroll
                        for (int j = 0; j < kRG - 1; ++j)
                            dd_x[j][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr_x[j][q][s], bw, z,
                                                                                0, 0, 0);
                    }
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float d = (float)as_h2(sw[q][s >> 1])[s & 1];   // v_fma_mix operand
#pragma unroll
                    for (int k = 0; k < kLive; ++k) {
                        acc[k] = __builtin_fmaf(d, dd[s][k], acc[k]);
                        if constexpr (kRG > 1) {
#pragma unroll
                            for (int j = 0; j < kRG - 1; ++j)
                                acc_x[j][k] = __builtin_fmaf(d, dd_x[j][s][k], acc_x[j][k]);
                        }
                    }
                }
            }
            if (next) load_group(t + 1, q);
        }
        // undo the activation scale (a power of two: the products are exact)
        // and add each row's low part to its high part: paired, in the lane;
        // one row, from lanes 32..63 (slot 8) to lanes 0..31 (slot 0)
        if constexpr (kPair) {
#pragma unroll
            for (int u = 0; u < kRpg; ++u) {
                const int row = g * kRpg + u;
                const float v = acc[2 * u] * inv[2 * u] + acc[2 * u + 1] * inv[2 * u + 1];
                if (row < NT) red[slot][wave][row][r] = v;
            }
        } else {
            float v[kLive];
#pragma unroll
            for (int i = 0; i < kLive; ++i) {
                v[i] = acc[i] * inv[i];
                if constexpr (kSplit) v[i] += __shfl_xor(v[i], 32);
            }
            if (!kSplit || g < 2) {
#pragma unroll
                for (int i = 0; i < kLive; ++i)
                    if (4 * g + i < NT) red[slot][wave][4 * g + i][r] = v[i];
            }
        }
        if constexpr (kRG > 1) {
#pragma unroll
            for (int j = 0; j < kRG - 1; ++j)
#pragma unroll
                for (int i = 0; i < kLive; ++i) {
                    const int rj = 16 * (j + 1) + 4 * g + i;
                    if (rj < NT) red[slot][wave][rj][r] = acc_x[j][i] * inv_x[j][i];
                }
        }
    };

    // Sum the parked partial sums of tiles [t0, t0 + cnt) over the waves, in
    // wave order, and store them.
    auto flush = [&](int t0, int cnt) {
        __syncthreads();
        for (int e = tid; e < cnt * NT * 16; e += blockDim.x) {
            const int sl = e / (NT * 16);
            const int tt = (e >> 4) % NT, rr = e & 15;
            const int t = t0 + sl;
            float sum = 0.0f;
            for (int w = 0; w < nact; ++w) sum += red[sl][w][tt][rr];
            if (!split) {
                const int row = t * kTileRows + rr;
                if (row < a.out && tt < args.nrows) {
                    if (bad_route) sum = __builtin_nanf("");
                    const int64_t yr = yslots ? yslots[tt] : tt;   // padding: -1
                    if (a.y && yr >= 0) a.y[yr * a.out + row] = sum;
                    if constexpr (NT <= kArgmaxRows) {
#pragma unroll
                        for (int u = 0; u < NT; ++u)
                            if (u == tt) amax_update(sum, row, bv[u], bi[u]);
                    }
                }
            } else {
                a.part[(((int64_t)sy * a.tiles + t) * kMaxRows + tt) * 16 + rr] =
                    bad_route ? __builtin_nanf("") : sum;
            }
        }
        __syncthreads();
    };

    // The loop body requests the next tile's words unconditionally and the
    // last tile is peeled, so the memory counter's order is the same on every
    // path and each product waits for its own words only.  Partial sums are
    // stored inside the loop only when a run exceeds kRedTiles tiles.
    int t0 = tb, t = tb;
    for (; t + 1 < te; ++t) {
        if (!idle) tile(t, t - t0, true);
        if (t - t0 == kRedTiles - 1) {
            flush(t0, kRedTiles);
            t0 = t + 1;
        }
    }
    if (!idle) tile(t, t - t0, false);
    flush(t0, t - t0 + 1);
    if constexpr (NT <= kArgmaxRows)
        if (a.amax && !split) amax_workgroup<NT>(bv, bi, a.amax + (int64_t)local * NT);
}

// Sum of the parked per-tile sums over the S slices, in slice order, for
// every split linear of a launch (flat element ranges, one after another).
struct ReduceLinear {
    const float *part;
    float *y;
    int64_t out, tiles, slices;
    int64_t e0;          // first flat element of this linear
};
struct ReduceArgs {
    ReduceLinear lin[kMaxGroupLinears];
    int nlin;
    int nrows;           // activation rows of the launch
    // routed launch: lin[0] per pair, pair_elems flat elements each, its
    // partial sums part_pair floats and its y row out floats further on
    int64_t pair_elems;
    int64_t part_pair;
    const int32_t *slot_pair;   // by expert: y row of each chunk row (-1: padding)
    int64_t total;
    uint2 *amax;         // per-workgroup (max, index) pairs of a single linear, or null
};

constexpr int kReduceBatch = 8;   // slice loads in flight per thread
template <int NT>
__global__ __launch_bounds__(256) void gemv_mfma_reduce_kernel(const ReduceArgs args) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    constexpr int kAm = NT <= kArgmaxRows ? NT : 1;
    float bv[kAm];
    int bi[kAm];
#pragma unroll
    for (int t = 0; t < kAm; ++t) {
        bv[t] = -__builtin_huge_valf();
        bi[t] = 0x7fffffff;
    }
    for (int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; f < args.total;
         f += stride) {
        int li = 0;
        for (int k = 1; k < args.nlin; ++k)
            if (f >= args.lin[k].e0) li = k;
        ReduceLinear L = args.lin[li];
        int64_t e = f - L.e0;
        int64_t chunk = 0;
        if (args.pair_elems > 0) {                   // routed: pair (chunk) of element f
            const int64_t pair = e / args.pair_elems;
            e -= pair * args.pair_elems;
            L.part += pair * args.part_pair;
            if (args.slot_pair) chunk = pair;
            else L.y += pair * L.out;
        }
        const int rr = (int)(e & 15);
        const int tt = (int)((e >> 4) % NT);
        const int64_t t = (e >> 4) / NT;
        // the slices' loads are issued in batches (indices past the last
        // slice re-read it and are not added), then added in slice order
        float s = 0.0f;
        for (int64_t q0 = 0; q0 < L.slices; q0 += kReduceBatch) {
            float v[kReduceBatch];
#pragma unroll
            for (int b = 0; b < kReduceBatch; ++b) {
                const int64_t q = q0 + b < L.slices ? q0 + b : L.slices - 1;
                v[b] = L.part[((q * L.tiles + t) * kMaxRows + tt) * 16 + rr];
            }
#pragma unroll
            for (int b = 0; b < kReduceBatch; ++b) s += q0 + b < L.slices ? v[b] : 0.0f;
        }
        const int64_t row = t * kTileRows + rr;
        if (row < L.out && tt < args.nrows) {
            const int64_t yr = args.slot_pair ? args.slot_pair[chunk * kChunkRows + tt] : tt;
            if (L.y && yr >= 0) L.y[yr * L.out + row] = s;
            if constexpr (NT <= kArgmaxRows) {
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    if (u == tt) amax_update(s, (int)row, bv[u], bi[u]);
            }
        }
    }
    if constexpr (NT <= kArgmaxRows)
        if (args.amax) amax_workgroup<NT>(bv, bi, args.amax + (int64_t)blockIdx.x * NT);
}

// Final (max, index) of each row of y over `count` workgroup pairs; row t's
// result in max_val[t], max_idx[t] (index -1 and a NaN value when no output
// of the row is a number).
template <int NT>
__global__ __launch_bounds__(256) void amax_final_kernel(const uint2 *__restrict__ pairs,
                                                         int count, float *max_val,
                                                         int32_t *max_idx) {
    float bv[NT];
    int bi[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        bv[t] = -__builtin_huge_valf();
        bi[t] = 0x7fffffff;
    }
    for (int k = threadIdx.x; k < count; k += blockDim.x)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint2 p = pairs[(int64_t)k * NT + t];
            amax_update(__builtin_bit_cast(float, p.x), (int)p.y, bv[t], bi[t]);
        }
    __shared__ uint2 res[NT];
    amax_workgroup<NT>(bv, bi, res);
    __syncthreads();
    if ((int)threadIdx.x < NT) {
        const int t = threadIdx.x;
        const bool none = (int)res[t].y == 0x7fffffff;
        max_val[t] = none ? __builtin_nanf("") : __builtin_bit_cast(float, res[t].x);
        max_idx[t] = none ? -1 : (int32_t)res[t].y;
    }
}

static int64_t mfma_lds_bytes(int64_t n, int64_t groups) {
    return groups * 4 * slots_for(n) * 64;
}

static int64_t round256(int64_t b) { return (b + 255) & ~(int64_t)255; }

// Bytes of the prepared fragments of an [n x in] x (header included).
static int64_t frag_bytes(int64_t n, int64_t in) {
    const Layout L(1, in);
    return round256(kFragHeader + L.g4 * 4 * slots_for(n) * 64);
}

// Whether a launch with n rows against an [out x in] matrix uses the pre-pass.
// A by-expert launch (gathered) always does: its pre-pass gathers each
// chunk's x rows through the routing plan.
static bool use_prep(int64_t n, int64_t out, int64_t in, bool gathered = false) {
    if (frag_bytes(n, in) > (int64_t)(kWorkspaceBytes / 4)) return false;
    if (gathered || n >= kPrepMinN) return true;
    return n >= kPrepMinNLarge && Layout(out, in).tiles >= kMfmaManyTiles;
}

static int gpw_for(int64_t per, int64_t n, bool prep) {
    for (int v : kGpwSet)
        if (v >= per && (prep || ((int64_t)v * 16 * stage_rows(n) + 63) / 64 <= kMaxStageItems))
            return v;
    return 0;
}

static MfmaPlan mfma_plan(int64_t n, int64_t out, int64_t in, bool gathered = false) {
    const Layout L(out, in);
    const bool prep = use_prep(n, out, in, gathered);
    n = kernel_rows(n);
    MfmaPlan p;
    // groups a wave may hold: the x it stages must fit its registers, or, when
    // prepared, the A fragments of its range
    int64_t per_cap = prep ? prep_groups(n) : (kMaxStageItems * 64) / (16 * stage_rows(n));
    if (per_cap > 16) per_cap = 16;
    if (per_cap < 1) per_cap = 1;     // n > 16: no plan can run (gemv_mfma_supports)
    // slices: as few as keep the slice within the waves' capacity and, when
    // x is staged in LDS, its A fragments within the LDS budget
    int64_t gps_max = per_cap * kMfmaMaxWaves;
    if (!prep && kMfmaLdsBudget / mfma_lds_bytes(n, 1) < gps_max)
        gps_max = kMfmaLdsBudget / mfma_lds_bytes(n, 1);
    if (gps_max < 1) gps_max = 1;
    p.slices = (L.g4 + gps_max - 1) / gps_max;
    p.gps = (L.g4 + p.slices - 1) / p.slices;
    // about Q4_MFMA_GROUPS_PER_WAVE groups per wave, at most kMfmaMaxWaves
    // waves; the register capacity rounds up to a compiled size
    int64_t waves = (p.gps + Q4_MFMA_GROUPS_PER_WAVE - 1) / Q4_MFMA_GROUPS_PER_WAVE;
    const int64_t min_waves = (p.gps + per_cap - 1) / per_cap;
    if (waves < min_waves) waves = min_waves;
    if (waves > kMfmaMaxWaves) waves = kMfmaMaxWaves;
    if (waves < 1) waves = 1;
    p.per = (int)((p.gps + waves - 1) / waves);
    p.waves = (int)((p.gps + p.per - 1) / p.per);
    p.gpw = gpw_for(p.per, n, prep);
    // about target_wgs() (or, for fewer tile-slices, target_wgs_small())
    // workgroups in all, each walking a run of tiles
    const int64_t units = L.tiles * p.slices;
    const int64_t target = units >= kMfmaManyTiles ? target_wgs() : target_wgs_small();
    int64_t tpw = (units + target - 1) / target;
    if (tpw < 1) tpw = 1;
    p.tpw = tpw;
    p.gx = (L.tiles + tpw - 1) / tpw;
    p.lds = prep ? 0 : (int64_t)p.waves * mfma_lds_bytes(n, p.per);
    return p;
}

static size_t mfma_part_bytes(const MfmaPlan &p, int64_t out, int64_t in) {
    if (p.slices == 1) return 0;
    const Layout L(out, in);
    return (size_t)round256(p.slices * L.tiles * kMaxRows * 16 * (int64_t)sizeof(float));
}

// (max, index) pairs of an argmax launch: one per row per workgroup of the
// kernel that finishes y (the product, or the K-slice reduction).
static int64_t amax_pairs(const MfmaPlan &p, int64_t n, int64_t out, int64_t in) {
    const Layout L(out, in);
    const int64_t wgs = p.slices == 1 ? p.gx : grid_for(L.tiles * n * 16, 256);
    return wgs * n;
}

// Launches above kMaxRows rows run as consecutive launches of up to
// kMaxRows rows each (the row slices of x and y), which read the weights
// once per slice; up to kMaxSlicedRows rows.
constexpr int64_t kMaxSlicedRows = 64;

static size_t launch_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    const size_t part = mfma_part_bytes(mfma_plan(n, out, in), out, in);
    return part + (use_prep(n, out, in) ? (size_t)frag_bytes(n, in) : 0);
}

static size_t launch_argmax_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    const MfmaPlan p = mfma_plan(n, out, in);
    return launch_workspace_bytes(n, out, in) +
           (size_t)round256(amax_pairs(p, n, out, in) * (int64_t)sizeof(uint2));
}

static bool launch_supported(int64_t n, int64_t out, int64_t in, bool gathered = false) {
    if (n < 1 || n > kMaxRows) return false;
    if (n > 16 && !use_prep(n, out, in, gathered)) return false;  // two A groups: prepared x
    const MfmaPlan p = mfma_plan(n, out, in, gathered);
    if (p.gpw == 0 || p.waves > kMfmaMaxWaves || p.slices > 65535) return false;
    if ((int64_t)p.waves * p.per < p.gps) return false;
    if (p.gx * p.slices > 0x7fffffff) return false;
    return launch_workspace_bytes(n, out, in) <= kWorkspaceBytes;
}

// Rows per launch for one matrix: launches of up to 64 rows read the weights
// once for all of them, but above 32 rows the K range is split (two groups
// per wave) and the partial sums travel through the workspace.  Measured on
// MI355X: FFN-up 9728 x 2560 at n = 48/64 22.4/25.9 us in one launch against
// 24.9/27.0 us in 32-row launches, the block grouped at n = 64 104.9 against
// 127.7 us; the 151936-row head at n = 64 237 us against 204 us.  So 64 rows
// per launch below kMfmaManyTiles tiles, 32 from there on.
static int64_t matrix_launch_rows(int64_t out, int64_t in) {
    return Layout(out, in).tiles >= kMfmaManyTiles ? 32 : kMaxRows;
}
int64_t gemv_mfma_launch_rows(const GemvProblem *probs, int count) {
    int64_t r = kMaxRows;
    for (int i = 0; i < count; ++i) {
        const int64_t ri = matrix_launch_rows(probs[i].out, probs[i].in);
        if (ri < r) r = ri;
    }
    return r;
}

// The row counts of the slices of an n-row call in launches of `rows`:
// full slices and the remainder (each slice's needs are those of its row
// count).
static int64_t tail_rows(int64_t n, int64_t rows) { return n % rows == 0 ? rows : n % rows; }

static size_t sliced_workspace_bytes(int64_t n, int64_t rows, int64_t out, int64_t in) {
    if (n <= rows) return launch_workspace_bytes(n, out, in);
    const size_t a = launch_workspace_bytes(rows, out, in);
    const size_t b = launch_workspace_bytes(tail_rows(n, rows), out, in);
    return a > b ? a : b;
}

// Covers both launch heights, so a group that runs a small matrix in the
// launches of a large one still fits.
size_t gemv_mfma_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    const size_t a = sliced_workspace_bytes(n, 32, out, in);
    const size_t b = sliced_workspace_bytes(n, kMaxRows, out, in);
    return a > b ? a : b;
}

size_t gemv_mfma_argmax_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    // greedy-pick calls run as launches of up to kArgmaxRows rows
    if (n <= kArgmaxRows) return launch_argmax_workspace_bytes(n, out, in);
    const size_t a = launch_argmax_workspace_bytes(kArgmaxRows, out, in);
    const size_t b = launch_argmax_workspace_bytes(tail_rows(n, kArgmaxRows), out, in);
    return a > b ? a : b;
}

static bool sliced_supported(int64_t n, int64_t rows, int64_t out, int64_t in) {
    if (n <= rows) return launch_supported(n, out, in);
    return launch_supported(rows, out, in) && launch_supported(tail_rows(n, rows), out, in);
}

bool gemv_mfma_supports(int64_t n, int64_t out, int64_t in, int x_f16) {
    (void)x_f16;
    if (n < 1 || n > kMaxSlicedRows) return false;
    // both launch heights: a group may run this matrix in either
    return sliced_supported(n, 32, out, in) && sliced_supported(n, kMaxRows, out, in);
}

bool gemv_mfma_group_uniform(const GemvProblem *probs, int count, int64_t n) {
    const int64_t lr = gemv_mfma_launch_rows(probs, count);
    // row slices decide the precision of x (high and low parts up to 8 rows),
    // so a group takes the slices each linear would take alone
    if (n > 32)
        for (int i = 0; i < count; ++i)
            if (matrix_launch_rows(probs[i].out, probs[i].in) != lr) return false;
    const int64_t rows[2] = {n < lr ? n : lr, tail_rows(n, lr)};
    for (int64_t r : rows)
        for (int i = 1; i < count; ++i)
            if (use_prep(r, probs[i].out, probs[i].in) != use_prep(r, probs[0].out, probs[0].in))
                return false;
    return true;
}

// Launches the instance if it exists (its groups fit the registers); returns
// whether it did.  idle: some linear of a grouped launch plans fewer waves
// than the launch has, so the IDLE instance runs (unprepared launches up to 8
// rows, where such groups arise: the block's seven linears in one call at
// n = 1/2/4 took 17.5/19.6/21.2 us with it against 23.6/25.0/22.0 us, the
// spare waves having requested their first group for every tile).
template <int NT, typename XT, int GPW, bool PREP>
static bool launch_mfma_g(bool idle, dim3 gd, dim3 bd, size_t lds, hipStream_t stream,
                          const GemvArgs &a) {
    if constexpr (PREP ? GPW <= prep_max_groups<NT>()
                       : (NT <= 16 &&
                          ((int64_t)GPW * 16 * stage_rows(NT) + 63) / 64 <= kMaxStageItems)) {
        if constexpr (!PREP && NT <= 8)
            if (idle) {
                hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, GPW, false, true>), gd, bd, lds,
                                   stream, a);
                return true;
            }
        hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, GPW, PREP, false>), gd, bd, lds, stream, a);
        return true;
    }
    return false;
}

template <int NT, typename XT, bool PREP>
static hipError_t launch_mfma_p(int gpw, bool idle, dim3 gd, dim3 bd, size_t lds,
                                hipStream_t stream, const GemvArgs &a) {
    bool launched = false;
    switch (gpw) {
    case 1: launched = launch_mfma_g<NT, XT, 1, PREP>(idle, gd, bd, lds, stream, a); break;
    case 2: launched = launch_mfma_g<NT, XT, 2, PREP>(idle, gd, bd, lds, stream, a); break;
    case 4: launched = launch_mfma_g<NT, XT, 4, PREP>(idle, gd, bd, lds, stream, a); break;
    case 5: launched = launch_mfma_g<NT, XT, 5, PREP>(idle, gd, bd, lds, stream, a); break;
    case 8:
        if (!PREP) launched = launch_mfma_g<NT, XT, 8, PREP>(idle, gd, bd, lds, stream, a);
        break;
    case 10:
        if (!PREP) launched = launch_mfma_g<NT, XT, 10, PREP>(idle, gd, bd, lds, stream, a);
        break;
    case 16:
        if (!PREP) launched = launch_mfma_g<NT, XT, 16, PREP>(idle, gd, bd, lds, stream, a);
        break;
    default: break;
    }
    if (!launched) return hipErrorInvalidValue;   // the plan asked for no compiled instance
    return hipGetLastError();
}

template <int NT, typename XT>
static hipError_t launch_mfma_t(const GemvProblem *probs, int count, void *ws,
                                hipStream_t stream, float *max_val, int32_t *max_idx,
                                int64_t nrows, const GemvRoute *route = nullptr,
                                int64_t npairs_routed = 0) {
    // the fused greedy pick runs launches of at most kArgmaxRows rows
    if (NT > kArgmaxRows && max_val) return hipErrorInvalidValue;
    // a routed launch: one linear (the experts' geometry), no pick
    if (route && (count != 1 || max_val || npairs_routed < 1)) return hipErrorInvalidValue;
    GemvArgs a = {};
    ReduceArgs ra = {};
    a.nrows = (int)nrows;
    ra.nrows = (int)nrows;
    int waves = 1, gpw = 0, min_waves = kMfmaMaxWaves;
    int64_t wg = 0, wsoff = 0;
    // by column: one unprepared row per pair; by expert: prepared chunks of kChunkRows rows
    const bool by_expert = route && route->chunk_expert;
    bool prep = true;
    // the linears of a group agree on the pre-pass (gemv_mfma_group_uniform)
    for (int i = 0; i < count; ++i)
        prep = prep && use_prep(nrows, probs[i].out, probs[i].in, by_expert);
    if (route && (by_expert ? (!prep || nrows != kChunkRows || NT != kChunkRows) : prep))
        return hipErrorInvalidValue;
    // a group: the weight groups of all its linears, for the shared target
    int64_t group_work = 0;
    if (count > 1)
        for (int i = 0; i < count; ++i) {
            const Layout Li(probs[i].out, probs[i].in);
            group_work += Li.tiles * Li.g4;
        }
    for (int i = 0; i < count; ++i) {
        const GemvProblem &pr = probs[i];
        MfmaPlan p = mfma_plan(nrows, pr.out, pr.in, by_expert);
        const Layout L(pr.out, pr.in);
        if (count > 1) {
            // this linear's share of the group's workgroups (the runs of
            // tiles change, not the sums: a tile's waves and K slices are
            // added in the same order whichever workgroup walks it)
            const int64_t units = L.tiles * p.slices;
            const int64_t total = (int64_t)device_shape().cus * Q4_MFMA_GROUP_WGS_PER_CU;
            int64_t target = (total * L.tiles * L.g4 + group_work - 1) / group_work;
            if (target < 1) target = 1;
            p.tpw = (units + target - 1) / target;
            p.gx = (L.tiles + p.tpw - 1) / p.tpw;
        }
        if (route) {
            // about Q4_MFMA_ROUTED_WGS_PER_CU workgroups per compute unit over
            // all pairs (chunks): each
            // workgroup stages or loads its pair's (chunk's) x once, so with
            // many pairs a pair takes few workgroups with long runs of tiles
            // (by column at 16 rows: 22.3 us against 27.4 us with the
            // one-linear plan's 48 workgroups per pair)
            int64_t gx = (int64_t)device_shape().cus * Q4_MFMA_ROUTED_WGS_PER_CU / npairs_routed;
            if (gx < 1) gx = 1;
            if (gx > L.tiles) gx = L.tiles;
            p.tpw = (L.tiles + gx - 1) / gx;
            p.gx = (L.tiles + p.tpw - 1) / p.tpw;
        }
        GemvLinear &g = a.lin[i];
        g.packed = (const uint8_t *)pr.packed;
        g.x = pr.x;
        g.y = pr.y;
        g.part = nullptr;
        g.frag = nullptr;
        g.amax = nullptr;
        if (p.slices > 1) {
            g.part = (float *)((uint8_t *)ws + wsoff);
            ReduceLinear &rl = ra.lin[ra.nlin++];
            rl.part = g.part;
            rl.y = pr.y;
            rl.out = pr.out;
            rl.tiles = L.tiles;
            rl.slices = p.slices;
            rl.e0 = ra.total;
            ra.total += L.tiles * NT * 16;
            const int64_t pb = (int64_t)mfma_part_bytes(p, pr.out, pr.in);
            if (route) {                            // each pair (chunk) its own partial sums
                ra.pair_elems = L.tiles * NT * 16;
                ra.part_pair = pb / (int64_t)sizeof(float);
                ra.slot_pair = by_expert ? route->slot_pair : nullptr;
                ra.total = ra.pair_elems * npairs_routed;
                wsoff += pb * npairs_routed;
            } else {
                wsoff += pb;
            }
        }
        g.code_base = L.scale_bytes();
        g.out = (int)pr.out;
        g.in = (int)pr.in;
        g.g4 = (int)L.g4;
        g.tiles = (int)L.tiles;
        g.gps = (int)p.gps;
        g.per = p.per;
        g.tpw = (int)p.tpw;
        g.gx = (int)p.gx;
        g.wg0 = (int)wg;
        wg += p.gx * p.slices;
        if (p.waves > waves) waves = p.waves;
        if (p.waves < min_waves) min_waves = p.waves;
        if (p.gpw > gpw) gpw = p.gpw;
    }
    a.nlin = count;
    if (route) {
        a.rt = *route;
        a.rt.wpp = (int)wg;                         // the one linear's workgroups
        a.rt.part_pair = ra.part_pair;
        wg *= npairs_routed;
    }
    // prepared launch: one pre-pass converting every distinct x of the group,
    // each x's fragments after the partial sums in the workspace
    if (prep) {
        PrepSet set = {};
        set.rows = (int)nrows;
        for (int i = 0; i < count; ++i) {
            for (int j = 0; j < i && !a.lin[i].frag; ++j)
                if (probs[j].x == probs[i].x && probs[j].in == probs[i].in)
                    a.lin[i].frag = a.lin[j].frag;
            if (a.lin[i].frag) continue;
            uint8_t *f = (uint8_t *)ws + wsoff;
            a.lin[i].frag = f;
            const int64_t fb = frag_bytes(nrows, probs[i].in);
            XRegions reg = {};
            int64_t units = 1;
            if (by_expert) {                        // every x row once, 8-row regions
                units = (route->x_rows + kChunkRows - 1) / kChunkRows;
                reg = {fb, route->x_rows};
                a.rt.frag_chunk = fb;
            }
            wsoff += fb * units;
            const int nbpad = a.lin[i].g4 * 4;
            // one workgroup per row of x (rows of the instance past nrows are
            // never read: their products land in outputs that are not stored)
            if (by_expert) {
                hipLaunchKernelGGL((route_prep_kernel<NT, XT>),
                                   dim3((unsigned)(1 + nrows * units)), dim3(kPrepThreads), 0,
                                   stream, route->route, route->x_rows * route->k,
                                   route->n_experts, (int)npairs_routed,
                                   (int32_t *)route->chunk_expert, (int32_t *)route->slot_pair,
                                   (const XT *)probs[i].x, (int)probs[i].in, nbpad, f, reg);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
            } else {
                set.x[set.count] = probs[i].x;
                set.frag[set.count] = f;
                set.in[set.count] = (int)probs[i].in;
                set.nbpad[set.count] = nbpad;
                ++set.count;
            }
        }
        if (set.count > 0) {
            hipLaunchKernelGGL((xprep_kernel<NT, XT>), dim3((unsigned)(nrows * set.count)),
                               dim3(kPrepThreads), 0, stream, set);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    // each wave's fragment region is laid out with its own linear's `per`;
    // the dynamic LDS covers the largest plan (waves x per x fragment bytes)
    int64_t lds = 0;
    if (!prep)
        for (int i = 0; i < count; ++i) {
            const int64_t b = (int64_t)waves * mfma_lds_bytes(NT, a.lin[i].per);
            if (b > lds) lds = b;
        }
    // argmax of a single linear: (max, index) pairs after everything else
    uint2 *pairs = nullptr;
    int npairs = 0;
    if (max_val) {
        pairs = (uint2 *)((uint8_t *)ws + wsoff);
        if (ra.nlin == 0) {
            a.lin[0].amax = pairs;
            npairs = a.lin[0].gx;
        } else {
            ra.amax = pairs;
            npairs = (int)grid_for(ra.total, 256);
        }
    }
    const dim3 gd((unsigned)wg), bd(waves * 64);
    const bool idle = count > 1 && min_waves < waves;
    hipError_t e;
    if constexpr (NT > 16)
        e = prep ? launch_mfma_p<NT, XT, true>(gpw, false, gd, bd, (size_t)lds, stream, a)
                 : hipErrorInvalidValue;
    else
        e = prep ? launch_mfma_p<NT, XT, true>(gpw, false, gd, bd, (size_t)lds, stream, a)
                 : launch_mfma_p<NT, XT, false>(gpw, idle, gd, bd, (size_t)lds, stream, a);
    if (e != hipSuccess) return e;
    if (ra.nlin > 0) {
        hipLaunchKernelGGL((gemv_mfma_reduce_kernel<NT>),
                           dim3((unsigned)grid_for(ra.total, 256)), dim3(256), 0, stream, ra);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!max_val) return hipSuccess;
    if constexpr (NT <= kArgmaxRows) {
        hipLaunchKernelGGL((amax_final_kernel<NT>), dim3(1), dim3(256), 0, stream,
                           (const uint2 *)pairs, npairs, max_val, max_idx);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <typename XT>
static hipError_t launch_mfma_x(const GemvProblem *probs, int count, int64_t n, void *ws,
                                hipStream_t stream, float *mv, int32_t *mi) {
    switch (n) {
    case 1: return launch_mfma_t<1, XT>(probs, count, ws, stream, mv, mi, n);
    case 2: return launch_mfma_t<2, XT>(probs, count, ws, stream, mv, mi, n);
    case 3: return launch_mfma_t<3, XT>(probs, count, ws, stream, mv, mi, n);
    case 4: return launch_mfma_t<4, XT>(probs, count, ws, stream, mv, mi, n);
    case 5: return launch_mfma_t<5, XT>(probs, count, ws, stream, mv, mi, n);
    case 6: return launch_mfma_t<6, XT>(probs, count, ws, stream, mv, mi, n);
    case 7: return launch_mfma_t<7, XT>(probs, count, ws, stream, mv, mi, n);
    case 8: return launch_mfma_t<8, XT>(probs, count, ws, stream, mv, mi, n);
    case 9: return launch_mfma_t<9, XT>(probs, count, ws, stream, mv, mi, n);
    case 10: return launch_mfma_t<10, XT>(probs, count, ws, stream, mv, mi, n);
    case 11: return launch_mfma_t<11, XT>(probs, count, ws, stream, mv, mi, n);
    case 12: return launch_mfma_t<12, XT>(probs, count, ws, stream, mv, mi, n);
    case 13: return launch_mfma_t<13, XT>(probs, count, ws, stream, mv, mi, n);
    case 14: return launch_mfma_t<14, XT>(probs, count, ws, stream, mv, mi, n);
    case 15: return launch_mfma_t<15, XT>(probs, count, ws, stream, mv, mi, n);
    case 16: return launch_mfma_t<16, XT>(probs, count, ws, stream, mv, mi, n);
    case 17: return launch_mfma_t<17, XT>(probs, count, ws, stream, mv, mi, n);
    case 18: return launch_mfma_t<18, XT>(probs, count, ws, stream, mv, mi, n);
    case 19: return launch_mfma_t<19, XT>(probs, count, ws, stream, mv, mi, n);
    case 20: return launch_mfma_t<20, XT>(probs, count, ws, stream, mv, mi, n);
    case 21: return launch_mfma_t<21, XT>(probs, count, ws, stream, mv, mi, n);
    case 22: return launch_mfma_t<22, XT>(probs, count, ws, stream, mv, mi, n);
    case 23: return launch_mfma_t<23, XT>(probs, count, ws, stream, mv, mi, n);
    case 24: return launch_mfma_t<24, XT>(probs, count, ws, stream, mv, mi, n);
    case 25: return launch_mfma_t<25, XT>(probs, count, ws, stream, mv, mi, n);
    case 26: return launch_mfma_t<26, XT>(probs, count, ws, stream, mv, mi, n);
    case 27: return launch_mfma_t<27, XT>(probs, count, ws, stream, mv, mi, n);
    case 28: return launch_mfma_t<28, XT>(probs, count, ws, stream, mv, mi, n);
    case 29: return launch_mfma_t<29, XT>(probs, count, ws, stream, mv, mi, n);
    case 30: return launch_mfma_t<30, XT>(probs, count, ws, stream, mv, mi, n);
    case 31: return launch_mfma_t<31, XT>(probs, count, ws, stream, mv, mi, n);
    case 32: return launch_mfma_t<32, XT>(probs, count, ws, stream, mv, mi, n);
    default:
        if (n <= 48) return launch_mfma_t<48, XT>(probs, count, ws, stream, mv, mi, n);
        if (n <= 64) return launch_mfma_t<64, XT>(probs, count, ws, stream, mv, mi, n);
        return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_mfma_group(const GemvProblem *probs, int count, int64_t n, int x_f16,
                                  void *ws, hipStream_t stream) {
    if (count < 1 || count > kMaxGroupLinears) return hipErrorInvalidValue;
    return x_f16 ? launch_mfma_x<_Float16>(probs, count, n, ws, stream, nullptr, nullptr)
                 : launch_mfma_x<float>(probs, count, n, ws, stream, nullptr, nullptr);
}

hipError_t launch_gemv_mfma_argmax(const void *packed, const void *x, int x_f16, float *y,
                                   int64_t n, int64_t out, int64_t in, float *max_val,
                                   int32_t *max_idx, void *ws, hipStream_t stream) {
    const int64_t esize = x_f16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < n; r0 += kArgmaxRows) {
        const int64_t nr = n - r0 < kArgmaxRows ? n - r0 : kArgmaxRows;
        const GemvProblem p = {packed, (const uint8_t *)x + r0 * in * esize,
                               y ? y + r0 * out : nullptr, out, in};
        const hipError_t e =
            x_f16 ? launch_mfma_x<_Float16>(&p, 1, nr, ws, stream, max_val + r0, max_idx + r0)
                  : launch_mfma_x<float>(&p, 1, nr, ws, stream, max_val + r0, max_idx + r0);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_mfma(const void *packed, const void *x, int x_f16, float *y, int64_t n,
                            int64_t out, int64_t in, void *ws, hipStream_t stream) {
    const int64_t esize = x_f16 ? 2 : 4;
    const int64_t lr = matrix_launch_rows(out, in);
    for (int64_t r0 = 0; r0 < n; r0 += lr) {
        const int64_t nr = n - r0 < lr ? n - r0 : lr;
        const GemvProblem p = {packed, (const uint8_t *)x + r0 * in * esize, y + r0 * out, out,
                               in};
        const hipError_t e = launch_gemv_mfma_group(&p, 1, nr, x_f16, ws, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Chunks a by-expert call may use: each bucket's last chunk may be partial.
static int64_t max_chunks(int64_t pairs, int64_t n_experts) {
    const int64_t buckets = n_experts + 1 < pairs ? n_experts + 1 : pairs;
    return (pairs + kChunkRows - 1) / kChunkRows + buckets;
}

// Workspace of a by-expert call: the plan's tables, per chunk its partial
// sums (K split), then the prepared fragments of x in 8-row regions.
static int64_t by_expert_table_bytes(int64_t chunks) {
    return round256(chunks * 4) + round256(chunks * kChunkRows * 4);
}
size_t gemv_mfma_by_expert_workspace_bytes(int64_t n, int64_t k, int64_t n_experts, int64_t out,
                                           int64_t in) {
    const int64_t c = max_chunks(n * k, n_experts);
    const MfmaPlan p = mfma_plan(kChunkRows, out, in, true);
    return (size_t)(by_expert_table_bytes(c) + c * (int64_t)mfma_part_bytes(p, out, in) +
                    (n + kChunkRows - 1) / kChunkRows * frag_bytes(kChunkRows, in));
}

bool gemv_mfma_by_expert_supports(int64_t n, int64_t k, int64_t n_experts, int64_t out,
                                  int64_t in) {
    const int64_t pairs = n * k;
    if (pairs < 1 || pairs > kPlanMaxPairs || n_experts < 1 || n_experts + 1 > kPlanMaxBuckets)
        return false;
    if (!launch_supported(kChunkRows, out, in, true) || !use_prep(kChunkRows, out, in, true))
        return false;
    const MfmaPlan p = mfma_plan(kChunkRows, out, in, true);
    return p.gx * p.slices * max_chunks(pairs, n_experts) <= 0x7fffffff &&
           gemv_mfma_by_expert_workspace_bytes(n, k, n_experts, out, in) <= kWorkspaceBytes;
}

hipError_t launch_gemv_mfma_by_expert(const void *experts, int64_t n_experts, const void *x,
                                      int x_f16, const int32_t *route, int64_t k, float *y,
                                      int64_t n, int64_t out, int64_t in, void *ws,
                                      hipStream_t stream) {
    const int64_t pairs = n * k, chunks = max_chunks(pairs, n_experts);
    int32_t *chunk_expert = (int32_t *)ws;
    int32_t *slot_pair = (int32_t *)((uint8_t *)ws + round256(chunks * 4));
    GemvRoute rt = {};
    rt.route = route;                     // read by the plan, in the pre-pass launch
    rt.chunk_expert = chunk_expert;
    rt.slot_pair = slot_pair;
    rt.expert_bytes = Layout(out, in).total_bytes();
    rt.x_row_bytes = in * (x_f16 ? 2 : 4);
    rt.n_experts = (int)n_experts;
    rt.k = (int)k;
    rt.x_rows = (int)n;
    void *rest = (uint8_t *)ws + by_expert_table_bytes(chunks);
    const GemvProblem p = {experts, x, y, out, in};
    return x_f16 ? launch_mfma_t<kChunkRows, _Float16>(&p, 1, rest, stream, nullptr, nullptr,
                                                       kChunkRows, &rt, chunks)
                 : launch_mfma_t<kChunkRows, float>(&p, 1, rest, stream, nullptr, nullptr,
                                                    kChunkRows, &rt, chunks);
}

// Routed (mixture of experts, by column): every (x row, expert) pair is a
// one-row product of its own, all pairs in one launch.
size_t gemv_mfma_routed_workspace_bytes(int64_t pairs, int64_t out, int64_t in) {
    return (size_t)pairs * mfma_part_bytes(mfma_plan(1, out, in), out, in);
}

bool gemv_mfma_routed_supports(int64_t pairs, int64_t out, int64_t in) {
    if (pairs < 1 || !launch_supported(1, out, in)) return false;
    const MfmaPlan p = mfma_plan(1, out, in);
    return p.gx * p.slices * pairs <= 0x7fffffff &&
           gemv_mfma_routed_workspace_bytes(pairs, out, in) <= kWorkspaceBytes;
}

hipError_t launch_gemv_mfma_routed(const void *experts, int64_t n_experts, const void *x,
                                   int x_f16, const int32_t *route, int64_t k, float *y,
                                   int64_t n, int64_t out, int64_t in, void *ws,
                                   hipStream_t stream) {
    GemvRoute rt = {};
    rt.route = route;
    rt.expert_bytes = Layout(out, in).total_bytes();
    rt.x_row_bytes = in * (x_f16 ? 2 : 4);
    rt.n_experts = (int)n_experts;
    rt.k = (int)k;
    const GemvProblem p = {experts, x, y, out, in};
    return x_f16 ? launch_mfma_t<1, _Float16>(&p, 1, ws, stream, nullptr, nullptr, 1, &rt, n * k)
                 : launch_mfma_t<1, float>(&p, 1, ws, stream, nullptr, nullptr, 1, &rt, n * k);
}

}  // namespace q4
