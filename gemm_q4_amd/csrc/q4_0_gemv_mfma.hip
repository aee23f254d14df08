// Small-n Q4_0 product on the matrix cores: y[n x out] = x . W^T for n <= 8.
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
//      x.  Before the split the workgroup scales each activation row of its K
//      slice by a power of two chosen from the row's largest |x| (no binary16
//      overflow, no underflow of the low part); the scale is undone exactly
//      on the partial sums.  The workgroup converts its slice of x once, into
//      LDS, laid out as A fragments (16 bytes per lane and block); lanes of
//      unused slots read nothing and feed zeros.
//   B: exact q - 8 in binary16, decoded straight from the repacked code word
//      the lane loaded (no LDS round trip).
//   D: lane l holds slots 4*(l/16)+i, i = 0..3, of weight row l%16; per block
//      acc += d * D in float32 (d is the row's binary16 scale).
// hi and lo slots of a row are summed with one cross-lane shuffle (xor 32).
//
// Work split.  Workgroup (cx, sy) owns a run of 16-row tiles and the sy-th of
// S slices of K; its waves take contiguous runs of `per` <= GPW 4-block groups
// of the slice, every tile of the run.  Order of requests: the workgroup's x
// first (small, shared by every workgroup, so it comes from L2), then all of
// the first tile's code and scale words, each wave's loads unconditionally
// (a wave with fewer than GPW groups repeats its first address), so that the
// memory counter lets every consumer wait for exactly its own words: x is
// staged while the weights are still in flight, and block b's product waits
// only for block b's word.  Each later tile's words are requested before the
// current tile is computed.  Per tile the waves' partials meet in LDS and are
// summed in a fixed order.  K is split (S > 1) only when the slice's A fragments would
// not fit the LDS budget; then each workgroup parks its per-tile sums in a
// workspace and a second small kernel adds the S slices in slice order.  The
// kernel boundary orders the two, so no device-wide fence or atomic is needed
// (on this multi-die part such a fence writes back and invalidates L2).
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

#ifndef Q4_MFMA_TARGET_WGS
#define Q4_MFMA_TARGET_WGS 1024      // about four workgroups per compute unit
#endif
#ifndef Q4_MFMA_LDS_BUDGET
#define Q4_MFMA_LDS_BUDGET (56 * 1024)
#endif
constexpr int kMfmaMaxWaves = 8;
constexpr int kMfmaTargetWgs = Q4_MFMA_TARGET_WGS;
constexpr int64_t kMfmaLdsBudget = Q4_MFMA_LDS_BUDGET;   // A fragments per workgroup
// x items (8 values) a thread stages: budget / 32 bytes per item / 256 threads
constexpr int kMaxItems = (int)(Q4_MFMA_LDS_BUDGET / 32 / 256);
#ifndef Q4_MFMA_STAGE_ITEMS
#define Q4_MFMA_STAGE_ITEMS 2
#endif
// x items a staging thread aims to hold (sets the number of staging waves)
constexpr int kStageItems = Q4_MFMA_STAGE_ITEMS;
// groups per wave a kernel instance holds in registers
constexpr int kGpwSet[] = {2, 4, 5, 8, 10, 16};

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

// Everything the kernel needs, computed on the host (no division on device).
struct MfmaArgs {
    const uint8_t *packed;
    const void *x;
    float *y;
    float *part;         // per-slice partial sums when S > 1
    int64_t code_base;   // byte offset of the code stream in `packed`
    int out, in;
    int g4, tiles;       // groups per padded row, 16-row tiles
    int gps;             // groups per K slice
    int per;             // groups per wave (<= GPW)
    int tpw;             // tiles per workgroup
    int sw;              // waves that stage x (the first sw); the others only stream weights
};

struct MfmaPlan {
    int stagers;      // waves that stage x
    int waves;        // waves per workgroup
    int gpw;          // register capacity per wave (template bound), >= per
    int per;          // groups per wave
    int64_t gps;      // groups per K slice
    int64_t slices;   // S: workgroups along K
    int64_t tpw;      // tiles per workgroup
    int64_t gx;       // workgroups along the tiles
};

// A-fragment store in LDS for one K slice: for block bl of the slice, slot
// index j in [0, 2*NT) (j < NT: high part of row j; j >= NT: low part of row
// j - NT) and quarter g, 16 bytes at ((bl * 2*NT + j) * 4 + g) * 16, holding
// the row's scaled values at k = 32*bl + 4g + {0, 2, 16, 18, 1, 3, 17, 19}
// (the slot order of decode_word_pairs).
template <int NT, typename XT, int GPW>
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void gemv_mfma_kernel(const MfmaArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ float red[2][kMfmaMaxWaves][8][16];
    __shared__ float rowmax[kMfmaMaxWaves][8];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int sy = blockIdx.y;
    const int gs0 = sy * a.gps;                              // first group of the slice
    const int gsn = a.g4 - gs0 < a.gps ? a.g4 - gs0 : a.gps;  // groups in the slice
    const int nbs = gsn * 4;                                 // blocks in the slice
    // this wave's groups of the slice: [q0, q0 + ng)
    const int q0 = wave * a.per;
    const int ng = gsn - q0 < 0 ? 0 : (gsn - q0 < a.per ? gsn - q0 : a.per);
    const int tb = (int)blockIdx.x * a.tpw;                  // < tiles by the grid
    const int te = tb + a.tpw < a.tiles ? tb + a.tpw : a.tiles;
    const XT *__restrict__ x = (const XT *)a.x;

    // ---- request the slice of x -------------------------------------------
    // item = (block bl, row t, quarter gq): the 8 values k = 32bl + 4gq +
    // {0..3} and 32bl + 16 + 4gq + {0..3}.
    const int k0 = gs0 * 128;                                // first k of the slice
    const int kin = a.in - k0 < nbs * 32 ? a.in - k0 : nbs * 32;
    const int items = nbs * NT * 4;
    // x is loaded and staged by the first a.sw waves only: the other waves
    // request their weight words at once, and no x wait of a staging wave
    // covers weight loads (the memory counter is per wave and in order)
    const bool stager = wave < a.sw;
    const int nstage = a.sw * 64;
    float xv[kMaxItems][8];
#pragma unroll
    for (int ii = 0; ii < kMaxItems; ++ii) {
        const int it = tid + ii * nstage;
        const int gq = it & 3;
        const int t = (it >> 2) % NT;
        const int bl = (it >> 2) / NT;
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[ii][k] = 0.0f;
        if (stager && it < items && bl * 32 < kin) {
            const XT *p = x + (int64_t)t * a.in + k0 + 32 * bl + 4 * gq;
            const float4 u = load_x4<XT>(p), v = load_x4<XT>(p + 16);
            xv[ii][0] = u.x; xv[ii][1] = u.y; xv[ii][2] = u.z; xv[ii][3] = u.w;
            xv[ii][4] = v.x; xv[ii][5] = v.y; xv[ii][6] = v.z; xv[ii][7] = v.w;
        }
    }

    // ---- request the first tile's code and scale words --------------------
    // Group q of the wave is slice group q0 + q; a wave with fewer than GPW
    // groups (or none) repeats a valid address of its slice.
    const int gw = ng > 0 ? gs0 + q0 : gs0;
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

    // ---- stage the slice of x as A fragments -------------------------------
    // The workgroup reduces each row's max |x| (through LDS), then each thread
    // scales its items, splits them into high and low binary16 parts and
    // writes them as fragments.
    float mloc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) mloc[t] = 0.0f;
#pragma unroll
    for (int ii = 0; ii < kMaxItems; ++ii) {
        const int it = tid + ii * nstage;
        const int t = (it >> 2) % NT;
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(xv[ii][k]));
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) mloc[tt] = t == tt ? fmaxf(mloc[tt], m) : mloc[tt];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float m = mloc[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) rowmax[wave][t] = m;
    }
    __syncthreads();
    float scale[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float m = 0.0f;
        for (int w = 0; w < a.sw; ++w) m = fmaxf(m, rowmax[w][t]);
        // largest |x| of the row lands in [2^14, 2^15)
        scale[t] = 1.0f;
        if (m > 0.0f && m <= 3.0e38f) {
            const int e = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
            scale[t] = pow2f(14 - e);
        }
    }
#pragma unroll
    for (int ii = 0; ii < kMaxItems; ++ii) {
        const int it = tid + ii * nstage;
        if (stager && it < items) {
            const int gq = it & 3;
            const int t = (it >> 2) % NT;
            const int bl = (it >> 2) / NT;
            float sc = scale[0];
#pragma unroll
            for (int tt = 1; tt < NT; ++tt) sc = t == tt ? scale[tt] : sc;
            _Float16 hi[8], lo[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float sv = xv[ii][k] * sc;
                hi[k] = (_Float16)sv;
                lo[k] = (_Float16)(sv - (float)hi[k]);
            }
            // order k = {0, 2, 16, 18, 1, 3, 17, 19} (+4gq): v index {0,2,4,6,1,3,5,7}
            const h8_t fh = h8_t{hi[0], hi[2], hi[4], hi[6], hi[1], hi[3], hi[5], hi[7]};
            const h8_t fl = h8_t{lo[0], lo[2], lo[4], lo[6], lo[1], lo[3], lo[5], lo[7]};
            *reinterpret_cast<h8_t *>(smem + ((bl * 2 * NT + t) * 4 + gq) * 16) = fh;
            *reinterpret_cast<h8_t *>(smem + ((bl * 2 * NT + NT + t) * 4 + gq) * 16) = fl;
        }
    }
    __syncthreads();

    // lane's A slot r: high part of row r (r < NT), low part of row r - 8
    // (8 <= r < 8 + NT).  Lanes of unused slots read slot 0's fragment: a D
    // row depends only on its own A row, and the rows of unused slots are
    // never read, so their contents do not matter (they stay finite).
    const int jslot = r < NT ? r : ((r >= 8 && r < 8 + NT) ? NT + (r - 8) : 0);
    constexpr int kFragStride = 2 * NT * 64;                 // bytes per block
    const uint8_t *afrag = smem + (jslot * 4 + g) * 16 + q0 * 4 * kFragStride;
    // D slots a lane can hold live: 4g+i for i < min(NT, 4)
    constexpr int kLive = NT < 4 ? NT : 4;
    // inverse scale of the row behind D slot 4g+i (slot m and m+8 are one row)
    float inv[kLive];
#pragma unroll
    for (int i = 0; i < kLive; ++i) {
        const int row = (4 * g + i) & 7;
        float sc = 1.0f;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) sc = row == tt ? scale[tt] : sc;
        inv[i] = pow2f(127 - (int)(__builtin_bit_cast(uint32_t, sc) >> 23));
    }
    const Magic mg = pinned_magic();

    // One tile: per group, four independent products (one per block), then
    // acc += d * D on the live slots; the waves' sums meet in LDS.
    int par = 0;
    // With `next` set, group q's words of tile t + 1 are requested into the
    // same registers as soon as group q of tile t has consumed them.
    auto tile = [&](int t, bool next) {
        float acc[kLive];
#pragma unroll
        for (int k = 0; k < kLive; ++k) acc[k] = 0.0f;
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (q < ng) {
                const uint8_t *ag = afrag + q * 4 * kFragStride;
                f4_t dd[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const h8_t av = *reinterpret_cast<const h8_t *>(ag + s * kFragStride);
                    uint32_t qd[4];
                    decode_word_pairs(cw[q][s], mg, qd);
                    const f4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
                    dd[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pack_h8(qd), z, 0, 0, 0);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float d = (float)as_h2(sw[q][s >> 1])[s & 1];   // v_fma_mix operand
#pragma unroll
                    for (int k = 0; k < kLive; ++k) acc[k] = __builtin_fmaf(d, dd[s][k], acc[k]);
                }
            }
            if (next) load_group(t + 1, q);
        }
        // undo the activation scale, add low parts (slots 8..15, lanes 32..63)
        // to high parts (slots 0..7, lanes 0..31)
        float v[kLive];
#pragma unroll
        for (int i = 0; i < kLive; ++i) {
            v[i] = acc[i] * inv[i];
            v[i] += __shfl_xor(v[i], 32);
        }
        if (g < 2) {
#pragma unroll
            for (int i = 0; i < kLive; ++i) red[par][wave][4 * g + i][r] = v[i];
        }
        __syncthreads();
        for (int e = tid; e < NT * 16; e += blockDim.x) {
            const int tt = e >> 4, rr = e & 15;
            float sum = 0.0f;
            for (int w = 0; w < nwaves; ++w) sum += red[par][w][tt][rr];
            if (gridDim.y == 1) {
                const int row = t * kTileRows + rr;
                if (row < a.out) a.y[(int64_t)tt * a.out + row] = sum;
            } else {
                a.part[(((int64_t)sy * a.tiles + t) * 8 + tt) * 16 + rr] = sum;
            }
        }
        par ^= 1;
    };

    int t = tb;
    for (; t + 1 < te; ++t) tile(t, true);
    tile(t, false);
}

// y[t][row] = sum over the S slices of the parked per-tile sums, in slice order.
template <int NT>
__global__ __launch_bounds__(256) void gemv_mfma_reduce_kernel(const float *__restrict__ part,
                                                               float *__restrict__ y,
                                                               int64_t out, int64_t tiles,
                                                               int64_t slices) {
    const int64_t total = tiles * NT * 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int rr = (int)(e & 15);
        const int tt = (int)((e >> 4) % NT);
        const int64_t t = (e >> 4) / NT;
        float s = 0.0f;
        for (int64_t q = 0; q < slices; ++q) s += part[((q * tiles + t) * 8 + tt) * 16 + rr];
        const int64_t row = t * kTileRows + rr;
        if (row < out) y[(int64_t)tt * out + row] = s;
    }
}

static int64_t mfma_lds_bytes(int64_t n, int64_t gps) { return gps * 4 * 2 * n * 4 * 16; }

static MfmaPlan mfma_plan(int64_t n, int64_t out, int64_t in) {
    const Layout L(out, in);
    MfmaPlan p;
    // slices: as few as keep the slice's A fragments within the LDS budget
    int64_t gps_max = kMfmaLdsBudget / mfma_lds_bytes(n, 1);
    if (gps_max < 1) gps_max = 1;
    p.slices = (L.g4 + gps_max - 1) / gps_max;
    p.gps = (L.g4 + p.slices - 1) / p.slices;
    // about five groups per wave (5.6 KB of words in flight per wave per
    // tile), at most eight waves; the register capacity rounds up to a
    // compiled size
    int64_t waves = (p.gps + 4) / 5;
    // enough threads to hold the slice of x while it is staged
    const int64_t items = p.gps * 4 * n * 4;
    const int64_t stage_waves = (items + kMaxItems * 64 - 1) / (kMaxItems * 64);
    if (waves < stage_waves) waves = stage_waves;
    if (waves > kMfmaMaxWaves) waves = kMfmaMaxWaves;
    if (waves < 1) waves = 1;
    p.per = (int)((p.gps + waves - 1) / waves);
    p.waves = (int)((p.gps + p.per - 1) / p.per);
    p.gpw = 0;
    for (int v : kGpwSet)
        if (p.gpw == 0 && v >= p.per) p.gpw = v;
    // staging waves: as few as hold the slice's x items in registers
    p.stagers = (int)((items + kStageItems * 64 - 1) / (kStageItems * 64));
    if (p.stagers < 1) p.stagers = 1;
    if (p.stagers > p.waves) p.stagers = p.waves;
    // about kMfmaTargetWgs workgroups in all, each walking a run of tiles
    int64_t tpw = (L.tiles * p.slices + kMfmaTargetWgs - 1) / kMfmaTargetWgs;
    if (tpw < 1) tpw = 1;
    p.tpw = tpw;
    p.gx = (L.tiles + tpw - 1) / tpw;
    return p;
}

size_t gemv_mfma_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    const MfmaPlan p = mfma_plan(n, out, in);
    if (p.slices == 1) return 0;
    const Layout L(out, in);
    return (size_t)p.slices * (size_t)L.tiles * 8 * 16 * sizeof(float);
}

bool gemv_mfma_supports(int64_t n, int64_t out, int64_t in, int x_f16) {
    (void)x_f16;
    if (n < 1 || n > 8) return false;
    const MfmaPlan p = mfma_plan(n, out, in);
    if (p.gpw == 0 || p.waves > kMfmaMaxWaves || p.slices > 65535 || p.gx > 0x7fffffff)
        return false;
    if ((int64_t)p.waves * p.per < p.gps) return false;
    if (p.gps * 4 * n * 4 > (int64_t)kMaxItems * p.stagers * 64) return false;
    return gemv_mfma_workspace_bytes(n, out, in) <= kWorkspaceBytes;
}

template <int NT, typename XT>
static hipError_t launch_mfma_t(const void *packed, const void *x, float *y, int64_t out,
                                int64_t in, void *ws, hipStream_t stream) {
    const MfmaPlan p = mfma_plan(NT, out, in);
    const Layout L(out, in);
    MfmaArgs a;
    a.packed = (const uint8_t *)packed;
    a.x = x;
    a.y = y;
    a.part = p.slices > 1 ? (float *)ws : nullptr;
    a.code_base = L.scale_bytes();
    a.out = (int)out;
    a.in = (int)in;
    a.g4 = (int)L.g4;
    a.tiles = (int)L.tiles;
    a.gps = (int)p.gps;
    a.per = p.per;
    a.tpw = (int)p.tpw;
    a.sw = p.stagers;
    const dim3 gd((unsigned)p.gx, (unsigned)p.slices), bd(p.waves * 64);
    const size_t lds = (size_t)mfma_lds_bytes(NT, p.gps);
    switch (p.gpw) {
    case 2: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 2>), gd, bd, lds, stream, a); break;
    case 4: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 4>), gd, bd, lds, stream, a); break;
    case 5: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 5>), gd, bd, lds, stream, a); break;
    case 8: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 8>), gd, bd, lds, stream, a); break;
    case 10: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 10>), gd, bd, lds, stream, a); break;
    case 16: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 16>), gd, bd, lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.slices == 1) return e;
    const int64_t total = L.tiles * NT * 16;
    hipLaunchKernelGGL((gemv_mfma_reduce_kernel<NT>), dim3((unsigned)grid_for(total, 256)),
                       dim3(256), 0, stream, (const float *)a.part, y, out, L.tiles, p.slices);
    return hipGetLastError();
}

template <typename XT>
static hipError_t launch_mfma_x(const void *packed, const void *x, float *y, int64_t n,
                                int64_t out, int64_t in, void *ws, hipStream_t stream) {
    switch (n) {
    case 1: return launch_mfma_t<1, XT>(packed, x, y, out, in, ws, stream);
    case 2: return launch_mfma_t<2, XT>(packed, x, y, out, in, ws, stream);
    case 3: return launch_mfma_t<3, XT>(packed, x, y, out, in, ws, stream);
    case 4: return launch_mfma_t<4, XT>(packed, x, y, out, in, ws, stream);
    case 5: return launch_mfma_t<5, XT>(packed, x, y, out, in, ws, stream);
    case 6: return launch_mfma_t<6, XT>(packed, x, y, out, in, ws, stream);
    case 7: return launch_mfma_t<7, XT>(packed, x, y, out, in, ws, stream);
    case 8: return launch_mfma_t<8, XT>(packed, x, y, out, in, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_mfma(const void *packed, const void *x, int x_f16, float *y, int64_t n,
                            int64_t out, int64_t in, void *ws, hipStream_t stream) {
    return x_f16 ? launch_mfma_x<_Float16>(packed, x, y, n, out, in, ws, stream)
                 : launch_mfma_x<float>(packed, x, y, n, out, in, ws, stream);
}

}  // namespace q4
