// Small-n Q4_0 product on the matrix cores: y[n x out] = x . W^T for n <= 8.
//
// Why MFMA for a memory-bound product: a vector-ALU dot costs about n + 1.25
// VALU operations per weight, more than the ~3.9 per weight that 70% of HBM
// bandwidth leaves on gfx950 once n reaches 4 or so (golem's card hits the
// same wall past a few columns, golem-server README "On the card").  Here the
// VALU only decodes (about 1.5 operations per weight, independent of n) and
// one v_mfma_f32_16x16x32_f16 per Q4_0 block does all n dot products at once.
//
// Operands of one MFMA (M = 16 activation slots, N = 16 weight rows, K = 32 =
// one Q4_0 block):
//   A: slot m < 8 holds the binary16 high part of activation row m, slot
//      8 + m its low part x - hi (also binary16).  hi + lo carries 22 bits of
//      x.  Before the split each wave scales its slice of x by a power of two
//      chosen from the slice's largest |x| (no binary16 overflow, no underflow
//      of the low part); the scale is undone exactly on the partial sums.
//   B: exact q - 8 in binary16, decoded straight from the repacked code word
//      the lane loaded (no LDS round trip).
//   D: lane l holds slots 4*(l/16)+i, i = 0..3, of weight row l%16; per block
//      acc += d * D in float32 (d is the row's binary16 scale).
// hi and lo slots of a row are summed with one cross-lane shuffle (xor 32).
//
// Work split.  Workgroup (cx, sy) owns a run of 16-row tiles and the sy-th of
// S slices of K; its W <= 8 waves cut the slice into <= 20 blocks each and
// keep their activation fragments in registers for the whole tile run.  Per
// tile the waves' partials meet in LDS and are summed in a fixed order.  With
// S > 1 each workgroup parks its per-tile sums in a workspace, and the last
// workgroup of the run to finish (counted with one device-scope atomic) adds
// the S slices in slice order and writes y: one dispatch, deterministic.
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

constexpr int kMfmaKB = 20;          // blocks per wave (multiple of 4)
constexpr int kMfmaGroups = kMfmaKB / 4;
constexpr int kMfmaMaxWaves = 8;
constexpr int kMfmaMaxSliceBlocks = kMfmaKB * kMfmaMaxWaves;   // 160
constexpr int kMfmaTargetWgs = 512;  // about two workgroups per compute unit

// 2^e with e clamped to the float32 normal range.
__device__ __forceinline__ float pow2f(int e) {
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// The eight activations a lane with quarter g needs from block b:
// k = 32b + 4g + {0..3} and 32b + 16 + 4g + {0..3} (two aligned vectors).
__device__ __forceinline__ void load_x8(const float *__restrict__ xr, int64_t b, int g,
                                        float v[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(xr + 32 * b + 4 * g);
    const float4 c = *reinterpret_cast<const float4 *>(xr + 32 * b + 16 + 4 * g);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
}
__device__ __forceinline__ void load_x8(const _Float16 *__restrict__ xr, int64_t b, int g,
                                        float v[8]) {
    const u2_t a = *reinterpret_cast<const u2_t *>(xr + 32 * b + 4 * g);
    const u2_t c = *reinterpret_cast<const u2_t *>(xr + 32 * b + 16 + 4 * g);
    const h2_t a0 = as_h2(a[0]), a1 = as_h2(a[1]), c0 = as_h2(c[0]), c1 = as_h2(c[1]);
    v[0] = (float)a0.x; v[1] = (float)a0.y; v[2] = (float)a1.x; v[3] = (float)a1.y;
    v[4] = (float)c0.x; v[5] = (float)c0.y; v[6] = (float)c1.x; v[7] = (float)c1.y;
}

struct MfmaPlan {
    int waves;        // waves per workgroup
    int bpw;          // blocks per wave (multiple of 4)
    int64_t bps;      // blocks per K slice (multiple of 4)
    int64_t slices;   // S
    int64_t tpw;      // tiles per workgroup
    int64_t gx;       // workgroups along the tiles
};

template <int NT, typename XT, int MAXW>
__global__ __launch_bounds__(MAXW * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemv_mfma_kernel(
    const uint8_t *__restrict__ packed, const XT *__restrict__ x, float *__restrict__ y,
    int64_t out, int64_t in, int bpw, int64_t bps, int64_t tiles_per_wg,
    float *__restrict__ part, uint32_t *__restrict__ counters) {
    __shared__ float red[2][MAXW][8][16];
    __shared__ int last_flag;
    const Layout L(out, in);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t slices = gridDim.y;
    const int64_t sy = blockIdx.y;
    const int64_t nbp = L.g4 * kGroupBlocks;    // blocks incl. zero padding
    const int64_t s0 = sy * bps;
    const int64_t s1 = s0 + bps < nbp ? s0 + bps : nbp;
    const int64_t b0 = s0 + (int64_t)wave * bpw;
    const int64_t b1 = b0 + bpw < s1 ? b0 + bpw : s1;   // multiple of 4

    // ---- activation fragments for this wave's K range (one pass) ------------
    // Loads are unconditional (clamped to valid addresses) so they issue
    // back to back; invalid values are masked afterwards.
    const int tok = r < 8 ? r : r - 8;          // A slot r -> activation row
    const bool live = tok < NT;
    const XT *xr = x + (int64_t)(live ? tok : 0) * in;
    float xv[kMfmaKB][8];
#pragma unroll
    for (int i = 0; i < kMfmaKB; ++i) {
        const int64_t b = b0 + i;
        load_x8(xr, b < L.nb ? b : L.nb - 1, g, xv[i]);
        const bool ok = live && b < b1 && b < L.nb;
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[i][k] = ok ? xv[i][k] : 0.0f;
    }
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kMfmaKB; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(xv[i][k]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // scale so that the largest |x| of the slice lands in [2^14, 2^15)
    float scale = 1.0f;
    if (mx > 0.0f && mx <= 3.0e38f) {
        const int e = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF) - 127;
        scale = pow2f(14 - e);
    }
    h8_t xa[kMfmaKB];
#pragma unroll
    for (int i = 0; i < kMfmaKB; ++i) {
        _Float16 h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float s = xv[i][k] * scale;
            const _Float16 hi = (_Float16)s;
            h[k] = r < 8 ? hi : (_Float16)(s - (float)hi);
        }
        xa[i] = h8_t{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
    }
    // inverse scale of the activation row behind D slot 4g+i (slot m and
    // m+8 belong to the same row and were scaled alike); exact, a power of 2
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t sb = __builtin_bit_cast(uint32_t, __shfl(scale, 4 * g + i));
        inv[i] = pow2f(127 - (int)(sb >> 23));
    }

    // ---- tiles --------------------------------------------------------------
    const int64_t tb = (int64_t)blockIdx.x * tiles_per_wg;
    int64_t te = tb + tiles_per_wg;
    if (te > L.tiles) te = L.tiles;
    // Code and scale words per 4-block group of the wave's range.
    u4_t cw[kMfmaGroups], cwn[kMfmaGroups];
    u2_t sw[kMfmaGroups], swn[kMfmaGroups];
    auto load_tile = [&](int64_t t, u4_t (&c)[kMfmaGroups], u2_t (&sc)[kMfmaGroups]) {
        const uint8_t *codes = packed + L.tile_codes(t) + (b0 >> 2) * kGroupCodeBytes + lane * 16;
        const uint8_t *scales = packed + L.tile_scales(t) + (b0 >> 2) * kGroupScaleBytes + r * 8;
#pragma unroll
        for (int q = 0; q < kMfmaGroups; ++q) {
            if (b0 + 4 * q < b1) {
                c[q] = load_u4(codes + q * kGroupCodeBytes);
                sc[q] = load_u2(scales + q * kGroupScaleBytes);
            }
        }
    };

    if (tb < te) load_tile(tb, cw, sw);
    int par = 0;
    for (int64_t t = tb; t < te; ++t) {
        if (t + 1 < te) load_tile(t + 1, cwn, swn);
        f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < kMfmaKB; ++i) {
            const int64_t b = b0 + i;
            if (b < b1) {
                const uint32_t word = cw[i >> 2][i & 3];
                const uint32_t dbits = (sw[i >> 2][(i & 3) >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                uint32_t qd[4];
                decode_word(word, qd);
                const f4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
                const f4_t dd =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i], pack_h8(qd), z, 0, 0, 0);
                const float d = half_bits_to_float(dbits);
                acc[0] = __builtin_fmaf(d, dd[0], acc[0]);
                acc[1] = __builtin_fmaf(d, dd[1], acc[1]);
                acc[2] = __builtin_fmaf(d, dd[2], acc[2]);
                acc[3] = __builtin_fmaf(d, dd[3], acc[3]);
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
        if (threadIdx.x < NT * 16) {
            const int tt = threadIdx.x >> 4, rr = threadIdx.x & 15;
            float s = 0.0f;
            for (int w = 0; w < nwaves; ++w) s += red[par][w][tt][rr];
            if (slices == 1) {
                const int64_t row = t * kTileRows + rr;
                if (row < out) y[(int64_t)tt * out + row] = s;
            } else {
                part[((sy * L.tiles + t) * 8 + tt) * 16 + rr] = s;
            }
        }
        par ^= 1;
        if (t + 1 < te) {
#pragma unroll
            for (int q = 0; q < kMfmaGroups; ++q) { cw[q] = cwn[q]; sw[q] = swn[q]; }
        }
    }
    if (slices == 1) return;

    // ---- K slices: the last workgroup of this tile run adds them up ---------
    __threadfence();                 // publish this slice's partials
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = atomicAdd(&counters[blockIdx.x], 1u);
        last_flag = done == (uint32_t)(slices - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();                 // see every other slice's partials
    for (int64_t t = tb; t < te; ++t) {
        if (threadIdx.x < NT * 16) {
            const int tt = threadIdx.x >> 4, rr = threadIdx.x & 15;
            float s = 0.0f;
            for (int64_t q = 0; q < slices; ++q)
                s += __hip_atomic_load(&part[((q * L.tiles + t) * 8 + tt) * 16 + rr],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int64_t row = t * kTileRows + rr;
            if (row < out) y[(int64_t)tt * out + row] = s;
        }
    }
    if (threadIdx.x == 0) counters[blockIdx.x] = 0u;   // ready for the next call
}

static MfmaPlan mfma_plan(int64_t out, int64_t in) {
    const Layout L(out, in);
    MfmaPlan p;
    // slices: enough that each fits 8 waves x 20 blocks; more when there are
    // too few tiles to give every compute unit work
    const int64_t nbp = L.g4 * kGroupBlocks;
    int64_t smin = (nbp + kMfmaMaxSliceBlocks - 1) / kMfmaMaxSliceBlocks;
    int64_t s = smin;
    if (L.tiles < kMfmaTargetWgs) {
        int64_t want = (kMfmaTargetWgs + L.tiles - 1) / L.tiles;
        const int64_t smax = L.g4;                     // at least a group per slice
        if (want > smax) want = smax;
        if (want > s) s = want;
    }
    int64_t bps = (nbp + s - 1) / s;
    bps = (bps + 3) / 4 * 4;
    s = (nbp + bps - 1) / bps;
    int w = (int)((bps + kMfmaKB - 1) / kMfmaKB);
    int64_t bpw = (bps + w - 1) / w;
    bpw = (bpw + 3) / 4 * 4;
    w = (int)((bps + bpw - 1) / bpw);
    p.waves = w;
    p.bpw = (int)bpw;
    p.bps = bps;
    p.slices = s;
    int64_t tpw = 1;
    if (s == 1) tpw = (L.tiles + kMfmaTargetWgs - 1) / kMfmaTargetWgs;
    if (tpw < 1) tpw = 1;
    p.tpw = tpw;
    p.gx = (L.tiles + tpw - 1) / tpw;
    return p;
}

size_t gemv_mfma_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    (void)n;
    const MfmaPlan p = mfma_plan(out, in);
    if (p.slices == 1) return 0;
    const Layout L(out, in);
    const size_t part = (size_t)p.slices * (size_t)L.tiles * 8 * 16 * sizeof(float);
    const size_t cnt = (size_t)p.gx * sizeof(uint32_t);
    return ws_round(part) + ws_round(cnt);
}

bool gemv_mfma_supports(int64_t n, int64_t out, int64_t in, int x_f16) {
    (void)x_f16;
    if (n < 1 || n > 8) return false;
    const MfmaPlan p = mfma_plan(out, in);
    return p.waves <= kMfmaMaxWaves && p.bpw <= kMfmaKB && p.slices <= 65535 &&
           p.gx <= 0x7fffffff && gemv_mfma_workspace_bytes(n, out, in) <= kWorkspaceBytes;
}

template <int NT, typename XT>
static hipError_t launch_mfma_t(const void *packed, const void *x, float *y, int64_t out,
                                int64_t in, void *ws, hipStream_t stream) {
    const MfmaPlan p = mfma_plan(out, in);
    const Layout L(out, in);
    float *part = nullptr;
    uint32_t *counters = nullptr;
    if (p.slices > 1) {
        part = (float *)ws;
        counters = (uint32_t *)((char *)ws +
                                ws_round((size_t)p.slices * L.tiles * 8 * 16 * sizeof(float)));
    }
    const dim3 gd((unsigned)p.gx, (unsigned)p.slices), bd(p.waves * 64);
    const uint8_t *pk = (const uint8_t *)packed;
    const XT *xx = (const XT *)x;
    if (p.waves <= 4)
        hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 4>), gd, bd, 0, stream, pk, xx, y, out, in,
                           p.bpw, p.bps, p.tpw, part, counters);
    else
        hipLaunchKernelGGL((gemv_mfma_kernel<NT, XT, 8>), gd, bd, 0, stream, pk, xx, y, out, in,
                           p.bpw, p.bps, p.tpw, part, counters);
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
