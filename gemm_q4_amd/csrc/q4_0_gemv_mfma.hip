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
// S slices of K; its waves take contiguous runs of at most GPW 4-block groups
// of the slice, every tile of the run.  Each wave requests all of its code and
// scale words of a tile at once, and the next tile's words before it computes
// the current one.  Per tile the waves' partials meet in LDS and are summed in
// a fixed order.  K is split (S > 1) only when the slice's A fragments would
// not fit the LDS budget; then each workgroup parks its per-tile sums in a
// workspace and a second small kernel adds the S slices in slice order.  The
// kernel boundary orders the two, so no device-wide fence or atomic is needed
// (on this multi-die part such a fence writes back and invalidates L2).
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

#ifndef Q4_MFMA_TARGET_WGS
#define Q4_MFMA_TARGET_WGS 2048      // about eight workgroups per compute unit
#endif
#ifndef Q4_MFMA_LDS_BUDGET
#define Q4_MFMA_LDS_BUDGET (56 * 1024)
#endif
constexpr int kMfmaMaxWaves = 8;
constexpr int kMfmaTargetWgs = Q4_MFMA_TARGET_WGS;
constexpr int64_t kMfmaLdsBudget = Q4_MFMA_LDS_BUDGET;   // A fragments per workgroup
// x items (8 values) a thread stages: budget / 32 bytes per item / 256 threads
constexpr int kMaxItems = (int)(Q4_MFMA_LDS_BUDGET / 32 / 256);

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

struct MfmaPlan {
    int waves;        // waves per workgroup
    int gpw;          // groups per wave (at most, template bound)
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
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void gemv_mfma_kernel(
    const uint8_t *__restrict__ packed, const XT *__restrict__ x, float *__restrict__ y,
    int64_t out, int64_t in, int64_t gps, int64_t tiles_per_wg, float *__restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ float red[2][kMfmaMaxWaves][8][16];
    __shared__ float rowmax[kMfmaMaxWaves][8];
    const Layout L(out, in);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t slices = gridDim.y;
    const int64_t sy = blockIdx.y;
    const int64_t gs0 = sy * gps;                            // first group of the slice
    const int64_t gs1 = gs0 + gps < L.g4 ? gs0 + gps : L.g4;
    const int nbs = (int)(gs1 - gs0) * 4;                    // blocks in the slice
    // this wave's groups of the slice: [q0, q1)
    const int per = (int)((gs1 - gs0 + nwaves - 1) / nwaves);
    const int q0 = wave * per;
    const int q1 = q0 + per < (int)(gs1 - gs0) ? q0 + per : (int)(gs1 - gs0);
    const int ng = q1 > q0 ? q1 - q0 : 0;

    const int64_t tb = (int64_t)blockIdx.x * tiles_per_wg;
    int64_t te = tb + tiles_per_wg;
    if (te > L.tiles) te = L.tiles;

    // ---- code and scale words of the wave's groups, per tile ---------------
    u4_t cw[GPW], cwn[GPW];
    u2_t sw[GPW], swn[GPW];
    auto load_tile = [&](int64_t t, u4_t (&c)[GPW], u2_t (&sc)[GPW]) {
        const uint8_t *codes = packed + L.tile_codes(t) + (gs0 + q0) * kGroupCodeBytes + lane * 16;
        const uint8_t *scales = packed + L.tile_scales(t) + (gs0 + q0) * kGroupScaleBytes + r * 8;
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (q < ng) {
                c[q] = load_u4(codes + q * kGroupCodeBytes);
                sc[q] = load_u2(scales + q * kGroupScaleBytes);
            }
        }
    };
    // the first tile's words go out before x is staged: both latencies overlap
    if (tb < te) load_tile(tb, cw, sw);

    // ---- stage the slice of x as A fragments -------------------------------
    // One pass over global memory: item = (block bl, row t, quarter gq) holds
    // the 8 values k = 32bl + 4gq + {0..3} and 32bl + 16 + 4gq + {0..3}; each
    // thread loads its items into registers, the workgroup reduces the per-row
    // max |x| (through LDS), and the same registers are then scaled, split into
    // high and low binary16 parts and written as fragments.
    const int64_t k0 = gs0 * 128;                            // first k of the slice
    const int kin = (int)((in - k0) < (int64_t)nbs * 32 ? (in - k0) : (int64_t)nbs * 32);
    const int items = nbs * NT * 4;
    float xv[kMaxItems][8];
    float mloc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) mloc[t] = 0.0f;
#pragma unroll
    for (int ii = 0; ii < kMaxItems; ++ii) {
        const int it = tid + ii * (int)blockDim.x;
        const int gq = it & 3;
        const int t = (it >> 2) % NT;
        const int bl = (it >> 2) / NT;
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[ii][k] = 0.0f;
        if (it < items && bl * 32 < kin) {
            const XT *p = x + (int64_t)t * in + k0 + 32 * bl + 4 * gq;
            const float4 a = load_x4<XT>(p), c = load_x4<XT>(p + 16);
            xv[ii][0] = a.x; xv[ii][1] = a.y; xv[ii][2] = a.z; xv[ii][3] = a.w;
            xv[ii][4] = c.x; xv[ii][5] = c.y; xv[ii][6] = c.z; xv[ii][7] = c.w;
        }
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
        for (int w = 0; w < nwaves; ++w) m = fmaxf(m, rowmax[w][t]);
        // largest |x| of the row lands in [2^14, 2^15)
        scale[t] = 1.0f;
        if (m > 0.0f && m <= 3.0e38f) {
            const int e = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
            scale[t] = pow2f(14 - e);
        }
    }
#pragma unroll
    for (int ii = 0; ii < kMaxItems; ++ii) {
        const int it = tid + ii * (int)blockDim.x;
        if (it < items) {
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
    const uint8_t *afrag = smem + (jslot * 4 + g) * 16;     // + bl * (2*NT*64)
    constexpr int kFragStride = 2 * NT * 64;
    // inverse scale of the row behind D slot 4g+i (slot m and m+8 are one row)
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (4 * g + i) & 7;
        float sc = 1.0f;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) sc = row == tt ? scale[tt] : sc;
        inv[i] = pow2f(127 - (int)(__builtin_bit_cast(uint32_t, sc) >> 23));
    }

    // ---- tiles --------------------------------------------------------------
    int par = 0;
    for (int64_t t = tb; t < te; ++t) {
        if (t + 1 < te) load_tile(t + 1, cwn, swn);
        f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (q < ng) {
                const uint8_t *ag = afrag + (q0 + q) * 4 * kFragStride;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const h8_t a = *reinterpret_cast<const h8_t *>(ag + s * kFragStride);
                    uint32_t qd[4];
                    decode_word_pairs(cw[q][s], qd);
                    const f4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const f4_t dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pack_h8(qd), z, 0, 0, 0);
                    const float d = (float)as_h2(sw[q][s >> 1])[s & 1];   // v_fma_mix operand
                    // D slot 4g+k: with n <= 4 only k < n can be live (slots
                    // 0..n-1 on g = 0 lanes, 8..8+n-1 on g = 2 lanes)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (NT > 4 || k < NT) acc[k] = __builtin_fmaf(d, dd[k], acc[k]);
                }
            }
        }
        // undo the activation scale, add low parts (slots 8..15, lanes 32..63)
        // to high parts (slots 0..7, lanes 0..31)
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = acc[i] * inv[i];
            v[i] += __shfl_xor(v[i], 32);
        }
        if (g < 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) red[par][wave][4 * g + i][r] = v[i];
        }
        __syncthreads();
        for (int e = tid; e < NT * 16; e += blockDim.x) {
            const int tt = e >> 4, rr = e & 15;
            float sum = 0.0f;
            for (int w = 0; w < nwaves; ++w) sum += red[par][w][tt][rr];
            if (slices == 1) {
                const int64_t row = t * kTileRows + rr;
                if (row < out) y[(int64_t)tt * out + row] = sum;
            } else {
                part[((sy * L.tiles + t) * 8 + tt) * 16 + rr] = sum;
            }
        }
        par ^= 1;
        if (t + 1 < te) {
#pragma unroll
            for (int q = 0; q < GPW; ++q) { cw[q] = cwn[q]; sw[q] = swn[q]; }
        }
    }
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
    // waves: 4, or 8 for long slices; groups per wave within the template bound
    p.waves = p.gps > 20 ? 8 : 4;
    int per = (int)((p.gps + p.waves - 1) / p.waves);
    p.gpw = per <= 2 ? 2 : per <= 5 ? 5 : per <= 8 ? 8 : per <= 12 ? 12 : 16;
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
    if (p.waves > kMfmaMaxWaves || p.slices > 65535 || p.gx > 0x7fffffff) return false;
    if ((int64_t)p.waves * p.gpw < p.gps) return false;
    if (p.gps * 4 * n * 4 > (int64_t)kMaxItems * p.waves * 64) return false;
    return gemv_mfma_workspace_bytes(n, out, in) <= kWorkspaceBytes;
}

template <int NT, typename XT>
static hipError_t launch_mfma_t(const void *packed, const void *x, float *y, int64_t out,
                                int64_t in, void *ws, hipStream_t stream) {
    const MfmaPlan p = mfma_plan(NT, out, in);
    const Layout L(out, in);
    float *part = p.slices > 1 ? (float *)ws : nullptr;
    const dim3 gd((unsigned)p.gx, (unsigned)p.slices), bd(p.waves * 64);
    const size_t lds = (size_t)mfma_lds_bytes(NT, p.gps);
    const uint8_t *pk = (const uint8_t *)packed;
    const XT *xx = (const XT *)x;
    switch (p.gpw) {
    case 2: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 2>), gd, bd, lds, stream, pk, xx, y, out, in, p.gps, p.tpw, part); break;
    case 5: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 5>), gd, bd, lds, stream, pk, xx, y, out, in, p.gps, p.tpw, part); break;
    case 8: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 8>), gd, bd, lds, stream, pk, xx, y, out, in, p.gps, p.tpw, part); break;
    case 12: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 12>), gd, bd, lds, stream, pk, xx, y, out, in, p.gps, p.tpw, part); break;
    default: hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 16>), gd, bd, lds, stream, pk, xx, y, out, in, p.gps, p.tpw, part); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.slices == 1) return e;
    const int64_t total = L.tiles * NT * 16;
    hipLaunchKernelGGL((gemv_mfma_reduce_kernel<NT>), dim3((unsigned)grid_for(total, 256)),
                       dim3(256), 0, stream, (const float *)part, y, out, L.tiles, p.slices);
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
