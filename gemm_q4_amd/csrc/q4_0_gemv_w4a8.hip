// W4A8: Q4_0 weights against int8 activations on the integer matrix cores.
//
// rembed "Architecture", section "int8 quantization": activations quantized
// to 8-bit integers, an integer dot product per output and an offset
// correction subtracted in the epilogue, checked bit for bit against an
// integer reference; goinfer primer ch. 10 "Which kernel runs is a runtime
// decision": the quantized dot on 8-bit integer dot-product hardware.
//
// Activations: one scale per 32 values of a row (the weights' block size),
// d = max |x| / 127 and q = x / d rounded to nearest, ties to even, both in
// float32 with correctly rounded division (q = 0 for a block whose d is not a
// positive finite number).  quantize_x8_kernel writes q [n x in] (int8) and
// d [n x in/32] (float32).
//
// Product, for n <= 16 activation rows per launch: one
// v_mfma_i32_16x16x32_i8 per Q4_0 block and 16-row tile.  A: lane l = 16g + r
// holds the int8 codes of activation row r at k = 4g..4g+3 and 4g+16..4g+19
// of the block (loaded once per wave for its K range and kept in registers;
// rows past n are zeros).  B: the same k of weight row r: the low nibbles
// (mask) and the high nibbles (shift, mask) of the lane's repacked code word,
// as unsigned codes 0..15.  D[m][c] = sum_k q_x q_w exactly in int32; the
// offset 8 comes off as 8 * S[m], S = the block's sum of row m's codes (the
// colSum correction of rembed's int8 path).  Per block and live slot
// acc += (d_w * d_x) * (D - 8 S) in float32.  Each wave computes S with the
// integer dot of its codes against ones and parks (d_x, S) of its range in
// its own LDS region, read back per block in the D layout.
//
// Work split as in the small-n binary16 kernel: workgroups own runs of 16-row
// tiles and one K slice; waves own runs of 4-block groups; per-tile partial
// sums meet in LDS in wave order; K is split across workgroups only when the
// slice exceeds the waves' register capacity, with a second kernel adding the
// slices in order.
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

namespace {

constexpr int kW8MaxWaves = 8;
constexpr int kW8MaxRows = 16;
constexpr int kW8Groups = 5;          // groups a wave holds (A: 8 registers each)
// Workgroups a launch aims for, per compute unit of the device: this many
// from kW8ManyTiles tile-slices on, one below (each workgroup walks a run of
// tiles with its activation codes, as in the binary16 small-n kernel).
#ifndef Q4_W8_WGS_PER_CU
#define Q4_W8_WGS_PER_CU 4
#endif
#ifndef Q4_W8_WGS_PER_CU_SMALL
#define Q4_W8_WGS_PER_CU_SMALL 1
#endif
constexpr int64_t kW8ManyTiles = 4096;
constexpr int kW8ReduceBatch = 8;     // slice loads in flight per thread
constexpr int kW8RedTiles = 2;

typedef int i4_t __attribute__((ext_vector_type(4)));

struct W8Args {
    const uint8_t *packed;
    const int8_t *q;
    const float *d;
    float *y;
    float *part;         // K-split partial sums, or null
    int64_t code_base;
    int out, in, nb;     // nb = in / 32
    int g4, tiles, gps, per, tpw, gx;
};

// one activation scale of a block: max |x| / 127, NaN if any value is NaN
__device__ __forceinline__ float block_amax(const float v[32]) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax || a != a) amax = a;
    }
    return amax;
}

template <typename XT>
__global__ __launch_bounds__(256) void quantize_x8_kernel(const XT *__restrict__ x, int64_t n,
                                                          int64_t in, int8_t *__restrict__ q,
                                                          float *__restrict__ d) {
    const int64_t nb = in / 32;
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (row, block)
    if (item >= n * nb) return;
    const XT *xb = x + item * 32;                     // row-major: item = t * nb + b
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = (float)xb[j];
    const float s = block_amax(v) / 127.0f;
    d[item] = s;
    const bool ok = s > 0.0f && s <= 3.4028234663852886e38f;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t u = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = ok ? (int)rintf(v[4 * j + k] / s) : 0;
            u |= ((uint32_t)c & 0xFFu) << (8 * k);
        }
        w[j] = u;
    }
    u4_t *qo = reinterpret_cast<u4_t *>(q + item * 32);
    qo[0] = u4_t{w[0], w[1], w[2], w[3]};
    qo[1] = u4_t{w[4], w[5], w[6], w[7]};
}

template <int NT, int GPW>
__global__ __launch_bounds__(kW8MaxWaves * 64) void gemv_w4a8_kernel(const W8Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // (d_x, S) per wave
    __shared__ float red[kW8RedTiles][kW8MaxWaves][NT][16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int sy = (int)blockIdx.x / a.gx;
    const int cx = (int)blockIdx.x - sy * a.gx;
    const int gs0 = sy * a.gps;
    const int gsn = a.g4 - gs0 < a.gps ? a.g4 - gs0 : a.gps;
    const int q0 = wave * a.per;
    const int ng = gsn - q0 < 0 ? 0 : (gsn - q0 < a.per ? gsn - q0 : a.per);
    const int tb = cx * a.tpw;
    const int te = tb + a.tpw < a.tiles ? tb + a.tpw : a.tiles;
    const int gw = ng > 0 ? gs0 + q0 : gs0;
    const bool split = a.part != nullptr;

    // ---- this lane's activation codes of the wave's range ---------------------
    // block b = 4 (gw + q) + s; blocks past in (padding of the last group) and
    // rows past n are zeros
    u2_t av[GPW][4];
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int b = 4 * (gw + (q < ng ? q : 0)) + s;
            av[q][s] = u2_t{0u, 0u};
            if (r < NT && b < a.nb) {
                const int8_t *p = a.q + (int64_t)r * a.in + 32 * b + 4 * g;
                av[q][s] = u2_t{*reinterpret_cast<const uint32_t *>(p),
                                *reinterpret_cast<const uint32_t *>(p + 16)};
            }
        }

    // ---- the first tile's code and scale words -----------------------------------
    const uint8_t *cbase = a.packed + a.code_base + (int64_t)gw * kGroupCodeBytes + lane * 16;
    const uint8_t *sbase = a.packed + (int64_t)gw * kGroupScaleBytes + r * 8;
    u4_t cw[GPW];
    u2_t sw[GPW];
    auto load_group = [&](int t, int q) {
        const int64_t j = (int64_t)t * a.g4 + (q < ng ? q : 0);
        cw[q] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(cbase + j * kGroupCodeBytes));
        sw[q] = __builtin_nontemporal_load(reinterpret_cast<const u2_t *>(sbase + j * kGroupScaleBytes));
    };
#pragma unroll
    for (int q = 0; q < GPW; ++q) load_group(tb, q);
    __builtin_amdgcn_sched_barrier(0);

    // ---- (d_x, S) of the wave's blocks, in the wave's LDS region --------------
    // slot (block bl of the range, row m): float d_x, int S at (bl * 16 + m) * 8
    uint8_t *ds = smem + wave * (a.per * 4 * 16 * 8);
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            int sum = __builtin_amdgcn_sdot4((int)av[q][s][0], 0x01010101, 0, false);
            sum = __builtin_amdgcn_sdot4((int)av[q][s][1], 0x01010101, sum, false);
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            const int b = 4 * (gw + (q < ng ? q : 0)) + s;
            if (g == 0 && q < ng) {
                const float dx = (r < NT && b < a.nb) ? a.d[(int64_t)r * a.nb + b] : 0.0f;
                *reinterpret_cast<u2_t *>(ds + ((4 * q + s) * 16 + r) * 8) =
                    u2_t{__builtin_bit_cast(uint32_t, dx), (uint32_t)sum};
            }
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    constexpr int kLive = NT < 4 ? NT : 4;
    const uint8_t *dsl = ds + (4 * g) * 8;           // rows 4g.. of a block slot

    auto tile = [&](int t, int slot, bool next) {
        float acc[kLive];
#pragma unroll
        for (int k = 0; k < kLive; ++k) acc[k] = 0.0f;
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            if (q < ng) {
                i4_t dd[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint32_t w = cw[q][s];
                    const u2_t bw = {w & 0x0F0F0F0Fu, (w >> 4) & 0x0F0F0F0Fu};
                    const i4_t z = {0, 0, 0, 0};
                    dd[s] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                        __builtin_bit_cast(long, av[q][s]), __builtin_bit_cast(long, bw), z, 0,
                        0, 0);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float dw = (float)as_h2(sw[q][s >> 1])[s & 1];
                    const u4_t p01 = *reinterpret_cast<const u4_t *>(dsl + (4 * q + s) * 128);
                    const u4_t p23 = *reinterpret_cast<const u4_t *>(dsl + (4 * q + s) * 128 + 16);
                    const uint32_t dxb[4] = {p01[0], p01[2], p23[0], p23[2]};
                    const int sb[4] = {(int)p01[1], (int)p01[3], (int)p23[1], (int)p23[3]};
#pragma unroll
                    for (int k = 0; k < kLive; ++k) {
                        const float f = dw * __builtin_bit_cast(float, dxb[k]);
                        acc[k] = __builtin_fmaf(f, (float)(dd[s][k] - 8 * sb[k]), acc[k]);
                    }
                }
            }
            if (next) load_group(t + 1, q);
        }
#pragma unroll
        for (int i = 0; i < kLive; ++i)
            if (4 * g + i < NT) red[slot][wave][4 * g + i][r] = acc[i];
    };

    auto flush = [&](int t0, int cnt) {
        __syncthreads();
        for (int e = tid; e < cnt * NT * 16; e += blockDim.x) {
            const int sl = e / (NT * 16);
            const int tt = (e >> 4) % NT, rr = e & 15;
            const int t = t0 + sl;
            float sum = 0.0f;
            for (int w = 0; w < nwaves; ++w) sum += red[sl][w][tt][rr];
            if (!split) {
                const int row = t * kTileRows + rr;
                if (row < a.out) a.y[(int64_t)tt * a.out + row] = sum;
            } else {
                a.part[(((int64_t)sy * a.tiles + t) * kW8MaxRows + tt) * 16 + rr] = sum;
            }
        }
        __syncthreads();
    };

    int t0 = tb, t = tb;
    for (; t + 1 < te; ++t) {
        tile(t, t - t0, true);
        if (t - t0 == kW8RedTiles - 1) {
            flush(t0, kW8RedTiles);
            t0 = t + 1;
        }
    }
    tile(t, t - t0, false);
    flush(t0, t - t0 + 1);
}

__global__ __launch_bounds__(256) void w4a8_reduce_kernel(const float *__restrict__ part,
                                                          float *__restrict__ y, int64_t n,
                                                          int64_t out, int64_t tiles,
                                                          int64_t slices) {
    const int64_t total = tiles * n * 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int rr = (int)(e & 15);
        const int64_t tt = (e >> 4) % n;
        const int64_t t = (e >> 4) / n;
        // the slices' loads in batches (indices past the last slice re-read
        // it and are not added), added in slice order
        float s = 0.0f;
        for (int64_t q0 = 0; q0 < slices; q0 += kW8ReduceBatch) {
            float v[kW8ReduceBatch];
#pragma unroll
            for (int b = 0; b < kW8ReduceBatch; ++b) {
                const int64_t q = q0 + b < slices ? q0 + b : slices - 1;
                v[b] = part[((q * tiles + t) * kW8MaxRows + tt) * 16 + rr];
            }
#pragma unroll
            for (int b = 0; b < kW8ReduceBatch; ++b) s += q0 + b < slices ? v[b] : 0.0f;
        }
        const int64_t row = t * kTileRows + rr;
        if (row < out) y[tt * out + row] = s;
    }
}

struct W8Plan {
    int waves, per;
    int64_t gps, slices, tpw, gx, lds;
};

W8Plan w8_plan(int64_t out, int64_t in) {
    const Layout L(out, in);
    W8Plan p;
    const int64_t gps_max = (int64_t)kW8Groups * kW8MaxWaves;
    p.slices = (L.g4 + gps_max - 1) / gps_max;
    p.gps = (L.g4 + p.slices - 1) / p.slices;
    int64_t waves = (p.gps + kW8Groups - 1) / kW8Groups;
    if (waves < 1) waves = 1;
    p.per = (int)((p.gps + waves - 1) / waves);
    p.waves = (int)((p.gps + p.per - 1) / p.per);
    const int64_t units = L.tiles * p.slices;
    const int64_t cus = device_shape().cus;
    const int64_t target =
        cus * (units >= kW8ManyTiles ? Q4_W8_WGS_PER_CU : Q4_W8_WGS_PER_CU_SMALL);
    int64_t tpw = (units + target - 1) / target;
    if (tpw < 1) tpw = 1;
    p.tpw = tpw;
    p.gx = (L.tiles + tpw - 1) / tpw;
    p.lds = (int64_t)p.waves * p.per * 4 * 16 * 8;
    return p;
}

template <int NT>
hipError_t launch_w8_t(const void *packed, const int8_t *q, const float *d, float *y,
                       int64_t out, int64_t in, void *ws, hipStream_t stream) {
    const W8Plan p = w8_plan(out, in);
    const Layout L(out, in);
    W8Args a;
    a.packed = (const uint8_t *)packed;
    a.q = q;
    a.d = d;
    a.y = y;
    a.part = p.slices > 1 ? (float *)ws : nullptr;
    a.code_base = L.scale_bytes();
    a.out = (int)out;
    a.in = (int)in;
    a.nb = (int)(in / 32);
    a.g4 = (int)L.g4;
    a.tiles = (int)L.tiles;
    a.gps = (int)p.gps;
    a.per = p.per;
    a.tpw = (int)p.tpw;
    a.gx = (int)p.gx;
    const dim3 gd((unsigned)(p.gx * p.slices)), bd(p.waves * 64);
    switch (p.per) {
    case 1: hipLaunchKernelGGL((gemv_w4a8_kernel<NT, 1>), gd, bd, p.lds, stream, a); break;
    case 2: hipLaunchKernelGGL((gemv_w4a8_kernel<NT, 2>), gd, bd, p.lds, stream, a); break;
    case 3: case 4:
        hipLaunchKernelGGL((gemv_w4a8_kernel<NT, 4>), gd, bd, p.lds, stream, a); break;
    case 5: hipLaunchKernelGGL((gemv_w4a8_kernel<NT, 5>), gd, bd, p.lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.slices == 1) return e;
    const int64_t total = L.tiles * NT * 16;
    hipLaunchKernelGGL(w4a8_reduce_kernel, dim3((unsigned)grid_for(total, 256)), dim3(256), 0,
                       stream, (const float *)a.part, y, (int64_t)NT, out, L.tiles, p.slices);
    return hipGetLastError();
}

}  // namespace

size_t w4a8_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    (void)n;
    const W8Plan p = w8_plan(out, in);
    if (p.slices == 1) return 0;
    const Layout L(out, in);
    return (size_t)p.slices * (size_t)L.tiles * kW8MaxRows * 16 * sizeof(float);
}

bool w4a8_supports(int64_t n, int64_t out, int64_t in) {
    if (n < 1 || n > 64) return false;
    const W8Plan p = w8_plan(out, in);
    if (p.gx * p.slices > 0x7fffffff || p.per > kW8Groups) return false;
    return w4a8_workspace_bytes(n, out, in) <= kWorkspaceBytes;
}

hipError_t launch_quantize_x8(const void *x, int x_f16, int8_t *q, float *d, int64_t n,
                              int64_t in, hipStream_t stream) {
    const int64_t items = n * (in / 32);
    const dim3 gd((unsigned)((items + 255) / 256)), bd(256);
    if (x_f16)
        hipLaunchKernelGGL((quantize_x8_kernel<_Float16>), gd, bd, 0, stream,
                           (const _Float16 *)x, n, in, q, d);
    else
        hipLaunchKernelGGL((quantize_x8_kernel<float>), gd, bd, 0, stream, (const float *)x, n,
                           in, q, d);
    return hipGetLastError();
}

hipError_t launch_gemv_w4a8(const void *packed, const int8_t *q, const float *d, float *y,
                            int64_t n, int64_t out, int64_t in, void *ws, hipStream_t stream) {
    for (int64_t r0 = 0; r0 < n; r0 += kW8MaxRows) {
        const int64_t nr = n - r0 < kW8MaxRows ? n - r0 : kW8MaxRows;
        const int8_t *qs = q + r0 * in;
        const float *dsl = d + r0 * (in / 32);
        float *ys = y + r0 * out;
        hipError_t e;
        switch (nr) {
#define Q4_W8_CASE(N) \
    case N: e = launch_w8_t<N>(packed, qs, dsl, ys, out, in, ws, stream); break;
            Q4_W8_CASE(1) Q4_W8_CASE(2) Q4_W8_CASE(3) Q4_W8_CASE(4) Q4_W8_CASE(5) Q4_W8_CASE(6)
            Q4_W8_CASE(7) Q4_W8_CASE(8) Q4_W8_CASE(9) Q4_W8_CASE(10) Q4_W8_CASE(11)
            Q4_W8_CASE(12) Q4_W8_CASE(13) Q4_W8_CASE(14) Q4_W8_CASE(15) Q4_W8_CASE(16)
#undef Q4_W8_CASE
        default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4
