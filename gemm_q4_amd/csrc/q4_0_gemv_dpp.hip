// Small-n Q4_0 product on the vector ALUs: y[n x out] = x . W^T for n <= 8.
//
// Decode is the memory-bound case (goinfer primer ch. 10, "What the kernels
// are"): every weight byte is read from HBM once for all n activation rows,
// the way golem's passes carry several conversations through one read of the
// weights (golem README, "Several conversations, one pass").
//
// Work split.  A workgroup of four waves owns TQ (1 or 2) consecutive 16-row
// tiles and all of K; wave w takes the 4-block groups j = w, w+4, ...  Lane l = g*16+r
// reads, per tile and group, the 16-byte word holding code bytes 4g..4g+3 of
// row r for four blocks (one coalesced 1 KB chunk per wave) and 8 bytes of
// row r's scales.  x is staged once per workgroup in LDS as float32; lanes
// with the same g read the same x addresses (LDS broadcast), and each x value
// read is reused for the TQ tiles.
//
// Arithmetic per weight: exact q - 8 in binary16 (see decode_word_pairs),
// then a mixed-precision FMA (binary16 weight x float32 activation, float32
// accumulate) per activation row, and one FMA per block and row to apply d.
// Reduction: the four lanes sharing a row are combined with cross-lane
// shuffles (xor 16, xor 32), the four waves through LDS.
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

constexpr int kDppThreads = 256;
constexpr int kDppWaves = kDppThreads / 64;
constexpr int64_t kDppMaxLds = 64 * 1024;

__device__ __forceinline__ float4 load_f4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
__device__ __forceinline__ float4 load_f4(const _Float16 *p) {
    const u2_t a = *reinterpret_cast<const u2_t *>(p);
    const h2_t a0 = as_h2(a[0]), a1 = as_h2(a[1]);
    return float4{(float)a0.x, (float)a0.y, (float)a1.x, (float)a1.y};
}

template <int NT, int TQ>
__device__ __forceinline__ void dpp_block(const float *__restrict__ xs, int in, int b, int g,
                                          const uint32_t (&word)[TQ], const float (&d)[TQ],
                                          const Magic &mg, float (&acc)[TQ][NT]) {
    // x values this lane needs: k = 32b + 4g + {0,1,2,3} and 32b + 16 + 4g + {0..3}
    float xv[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float4 a = *reinterpret_cast<const float4 *>(xs + t * in + 32 * b + 4 * g);
        const float4 c = *reinterpret_cast<const float4 *>(xs + t * in + 32 * b + 16 + 4 * g);
        xv[t][0] = a.x; xv[t][1] = a.y; xv[t][2] = a.z; xv[t][3] = a.w;
        xv[t][4] = c.x; xv[t][5] = c.y; xv[t][6] = c.z; xv[t][7] = c.w;
    }
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
        uint32_t q[4];
        decode_word_pairs(word[i], mg, q);
        // q pairs hold k offsets (0,2), (16,18), (1,3), (17,19) -> x slots
        const h2_t q0 = as_h2(q[0]), q1 = as_h2(q[1]), q2 = as_h2(q[2]), q3 = as_h2(q[3]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float p = (float)q0.x * xv[t][0];
            p = __builtin_fmaf((float)q0.y, xv[t][2], p);
            p = __builtin_fmaf((float)q1.x, xv[t][4], p);
            p = __builtin_fmaf((float)q1.y, xv[t][6], p);
            p = __builtin_fmaf((float)q2.x, xv[t][1], p);
            p = __builtin_fmaf((float)q2.y, xv[t][3], p);
            p = __builtin_fmaf((float)q3.x, xv[t][5], p);
            p = __builtin_fmaf((float)q3.y, xv[t][7], p);
            acc[i][t] = __builtin_fmaf(d[i], p, acc[i][t]);
        }
    }
}

template <int NT, int TQ, typename XT>
__global__ __launch_bounds__(kDppThreads) void gemv_dpp_kernel(
    const uint8_t *__restrict__ packed, const XT *__restrict__ x, float *__restrict__ y,
    int64_t out, int64_t in64) {
    // Groups a wave handles per batch; the batch's code and scale words are
    // loaded before the previous batch is computed (the first batch before
    // x is staged), so memory latency overlaps the staging and the math.
    constexpr int CH = TQ >= 4 ? 2 : 4;
    extern __shared__ float smem[];
    const Layout L(out, in64);
    const int in = (int)in64;
    const int inp = (int)L.g4 * kGroupBlocks * kBlockK;   // row stride, padded
    float *xs = smem;                    // [NT][inp], zero past in
    float *red = smem + NT * inp;        // [waves][TQ][NT][16]
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const Magic mg = pinned_magic();
    const int g = lane >> 4, r = lane & 15;
    const int64_t tile0 = (int64_t)blockIdx.x * TQ;
    const int ng = (int)L.g4;

    u4_t cw[CH][TQ], cwn[CH][TQ];
    u2_t sw[CH][TQ], swn[CH][TQ];
    // batch c0 covers the wave's groups j = wave + 4*(c0 + c), c < CH
    auto load_batch = [&](int c0, u4_t (&c)[CH][TQ], u2_t (&sc)[CH][TQ]) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int j = wave + kDppWaves * (c0 + k);
#pragma unroll
            for (int i = 0; i < TQ; ++i) {
                const int64_t t = tile0 + i;
                if (j < ng && t < L.tiles) {
                    // streamed once: non-temporal loads keep L2 for x
                    c[k][i] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(
                        packed + L.tile_codes(t) + (int64_t)j * kGroupCodeBytes + lane * 16));
                    sc[k][i] = __builtin_nontemporal_load(reinterpret_cast<const u2_t *>(
                        packed + L.tile_scales(t) + (int64_t)j * kGroupScaleBytes + r * 8));
                } else {
                    c[k][i] = u4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                    sc[k][i] = u2_t{0u, 0u};
                }
            }
        }
    };
    load_batch(0, cw, sw);

    // x rows staged as float32, four values per thread and step
    const int inp4 = inp / 4, in4 = in / 4;
#pragma unroll 4
    for (int i = tid; i < NT * inp4; i += kDppThreads) {
        const int t = i / inp4, k4 = i - t * inp4;
        float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (k4 < in4) v = load_f4(x + (int64_t)t * in + 4 * k4);
        *reinterpret_cast<float4 *>(xs + t * inp + 4 * k4) = v;
    }
    __syncthreads();

    float acc[TQ][NT];
#pragma unroll
    for (int i = 0; i < TQ; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = 0.0f;

    const int nmine = ng > wave ? (ng - wave + kDppWaves - 1) / kDppWaves : 0;
    for (int c0 = 0; c0 < nmine; c0 += CH) {
        const bool more = c0 + CH < nmine;
        if (more) load_batch(c0 + CH, cwn, swn);
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int j = wave + kDppWaves * (c0 + k);
            if (j < ng) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    uint32_t word[TQ];
                    float d[TQ];
#pragma unroll
                    for (int i = 0; i < TQ; ++i) {
                        word[i] = cw[k][i][s];
                        d[i] = half_bits_to_float((sw[k][i][s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
                    }
                    dpp_block<NT, TQ>(xs, inp, 4 * j + s, g, word, d, mg, acc);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int k = 0; k < CH; ++k)
#pragma unroll
                for (int i = 0; i < TQ; ++i) { cw[k][i] = cwn[k][i]; sw[k][i] = swn[k][i]; }
        }
    }

    // lanes r, r+16, r+32, r+48 share row r: combine across the four quarters
#pragma unroll
    for (int i = 0; i < TQ; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float v = acc[i][t];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[i][t] = v;
        }
    if (g == 0) {
#pragma unroll
        for (int i = 0; i < TQ; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                red[((wave * TQ + i) * NT + t) * 16 + r] = acc[i][t];
    }
    __syncthreads();
    for (int e = tid; e < TQ * NT * 16; e += kDppThreads) {
        const int rr = e & 15;
        const int t = (e >> 4) % NT;
        const int i = (e >> 4) / NT;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kDppWaves; ++w) s += red[w * TQ * NT * 16 + e];
        const int64_t row = (tile0 + i) * kTileRows + rr;
        if (row < out) y[(int64_t)t * out + row] = s;
    }
}

static int64_t dpp_lds_bytes(int64_t n, int64_t in, int tq) {
    const Layout L(1, in);
    return (n * L.g4 * kGroupBlocks * kBlockK + (int64_t)kDppWaves * tq * n * 16) * 4;
}

static int dpp_tq(int64_t n) { return n <= 2 ? 2 : 1; }

bool gemv_dpp_supports(int64_t n, int64_t out, int64_t in, int x_f16) {
    (void)out; (void)x_f16;
    return n >= 1 && n <= 8 && dpp_lds_bytes(n, in, dpp_tq(n)) <= kDppMaxLds;
}

template <int NT, int TQ, typename XT>
static hipError_t launch_dpp_t(const void *packed, const void *x, float *y, int64_t out,
                               int64_t in, hipStream_t stream) {
    const Layout L(out, in);
    const int64_t grid = (L.tiles + TQ - 1) / TQ;
    const size_t lds = (size_t)dpp_lds_bytes(NT, in, TQ);
    hipLaunchKernelGGL((gemv_dpp_kernel<NT, TQ, XT>), dim3((unsigned)grid), dim3(kDppThreads),
                       lds, stream, (const uint8_t *)packed, (const XT *)x, y, out, in);
    return hipGetLastError();
}

template <typename XT>
static hipError_t launch_dpp_x(const void *packed, const void *x, float *y, int64_t n,
                               int64_t out, int64_t in, hipStream_t stream) {
    switch (n) {
    case 1: return launch_dpp_t<1, 2, XT>(packed, x, y, out, in, stream);
    case 2: return launch_dpp_t<2, 2, XT>(packed, x, y, out, in, stream);
    case 3: return launch_dpp_t<3, 1, XT>(packed, x, y, out, in, stream);
    case 4: return launch_dpp_t<4, 1, XT>(packed, x, y, out, in, stream);
    case 5: return launch_dpp_t<5, 1, XT>(packed, x, y, out, in, stream);
    case 6: return launch_dpp_t<6, 1, XT>(packed, x, y, out, in, stream);
    case 7: return launch_dpp_t<7, 1, XT>(packed, x, y, out, in, stream);
    case 8: return launch_dpp_t<8, 1, XT>(packed, x, y, out, in, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_dpp(const void *packed, const void *x, int x_f16, float *y, int64_t n,
                           int64_t out, int64_t in, hipStream_t stream) {
    return x_f16 ? launch_dpp_x<_Float16>(packed, x, y, n, out, in, stream)
                 : launch_dpp_x<float>(packed, x, y, n, out, in, stream);
}

}  // namespace q4
