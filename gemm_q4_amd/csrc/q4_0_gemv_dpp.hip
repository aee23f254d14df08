// Small-n Q4_0 product on the vector ALUs: y[n x out] = x . W^T for n <= 8.
//
// Decode is the memory-bound case (goinfer primer ch. 10, "What the kernels
// are"): every weight byte is read from HBM once for all n activation rows,
// the way golem's passes carry several conversations through one read of the
// weights (golem README, "Several conversations, one pass").
//
// Work split.  A workgroup of four waves owns TQ consecutive 16-row tiles and
// all of K; wave w takes the 4-block groups j = w, w+4, ...  Lane l = g*16+r
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

template <int NT, int TQ>
__device__ __forceinline__ void dpp_block(const float *__restrict__ xs, int in, int b, int g,
                                          const uint32_t (&word)[TQ], const float (&d)[TQ],
                                          float (&acc)[TQ][NT]) {
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
        decode_word_pairs(word[i], q);
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
    extern __shared__ float smem[];
    const Layout L(out, in64);
    const int in = (int)in64;
    const int inp = (int)L.g4 * kGroupBlocks * kBlockK;   // row stride, padded
    float *xs = smem;                    // [NT][inp], zero past in
    float *red = smem + NT * inp;        // [waves][TQ][NT][16]
    const int tid = threadIdx.x;

    for (int i = tid; i < NT * inp; i += kDppThreads) {
        const int t = i / inp, k = i - t * inp;
        xs[i] = k < in ? to_f32(x[(int64_t)t * in + k]) : 0.0f;
    }
    __syncthreads();

    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t tile0 = (int64_t)blockIdx.x * TQ;

    float acc[TQ][NT];
#pragma unroll
    for (int i = 0; i < TQ; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = 0.0f;

    for (int j = wave; j < (int)L.g4; j += kDppWaves) {
        u4_t cw[TQ];
        u2_t sw[TQ];
#pragma unroll
        for (int i = 0; i < TQ; ++i) {
            const int64_t t = tile0 + i;
            if (t < L.tiles) {
                cw[i] = load_u4(packed + L.tile_codes(t) + (int64_t)j * kGroupCodeBytes + lane * 16);
                sw[i] = load_u2(packed + L.tile_scales(t) + (int64_t)j * kGroupScaleBytes + r * 8);
            } else {
                cw[i] = u4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                sw[i] = u2_t{0u, 0u};
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t word[TQ];
            float d[TQ];
#pragma unroll
            for (int i = 0; i < TQ; ++i) {
                word[i] = cw[i][s];
                d[i] = half_bits_to_float((sw[i][s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
            }
            dpp_block<NT, TQ>(xs, inp, 4 * j + s, g, word, d, acc);
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

static int dpp_tq(int64_t n) { return n <= 2 ? 4 : 2; }

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
    case 1: return launch_dpp_t<1, 4, XT>(packed, x, y, out, in, stream);
    case 2: return launch_dpp_t<2, 4, XT>(packed, x, y, out, in, stream);
    case 3: return launch_dpp_t<3, 2, XT>(packed, x, y, out, in, stream);
    case 4: return launch_dpp_t<4, 2, XT>(packed, x, y, out, in, stream);
    case 5: return launch_dpp_t<5, 2, XT>(packed, x, y, out, in, stream);
    case 6: return launch_dpp_t<6, 2, XT>(packed, x, y, out, in, stream);
    case 7: return launch_dpp_t<7, 2, XT>(packed, x, y, out, in, stream);
    case 8: return launch_dpp_t<8, 2, XT>(packed, x, y, out, in, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_dpp(const void *packed, const void *x, int x_f16, float *y, int64_t n,
                           int64_t out, int64_t in, hipStream_t stream) {
    return x_f16 ? launch_dpp_x<_Float16>(packed, x, y, n, out, in, stream)
                 : launch_dpp_x<float>(packed, x, y, n, out, in, stream);
}

}  // namespace q4
