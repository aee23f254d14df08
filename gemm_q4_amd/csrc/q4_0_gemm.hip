// Prefill Q4_0 product on the matrix cores: y[n x out] = x . W^T for large n.
//
// The compute-bound case (goinfer primer ch. 10, "What the kernels are": GEMM
// is prefill's workhorse; golem reads prompts in passes of up to 512
// positions, golem README "Reading a prompt on the card").
//
// Tile: a workgroup of four waves computes 64 activation rows x 256 weight
// rows; wave w owns weight rows [64w, 64w+64) of the tile (four 16-row tiles)
// against all 64 activation rows, as 4 x 4 accumulators of
// v_mfma_f32_16x16x32_f16 (one MFMA K step = one Q4_0 block).
//
// Operands per K step of four blocks (128 k):
//   x: 64 rows x 128 k of binary16, staged in LDS (double buffered) in MFMA
//      A-fragment order: for each row and block, the eight k-values a lane
//      with quarter g needs (4g..4g+3 and 4g+16..4g+19) are 16 contiguous
//      bytes, read with one ds_read_b128.  float32 activations are rounded to
//      binary16 when staged.
//   W: each lane loads its own 16-byte code word and 8-byte scale word per
//      16-row tile straight from the repacked stream (the word is the MFMA
//      B fragment), decodes exact q - 8 and multiplies by d in binary16, so
//      each weight is rounded once.  The next step's words are loaded before
//      the current step is computed.
#include "q4_0_device.h"
#include "q4_0_internal.h"

namespace q4 {

constexpr int kGemmBM = 64;                  // activation rows per workgroup
constexpr int kGemmBN = 256;                 // weight rows per workgroup
constexpr int kGemmWaves = 4;
constexpr int kGemmTilesPerWave = kGemmBN / kGemmWaves / kTileRows;  // 4
constexpr int kGemmMSub = kGemmBM / 16;      // 4
constexpr int kXRowBytes = 4 * 4 * 16 + 16;  // one row of a K step, padded

template <typename XT>
__device__ __forceinline__ void load_x_piece(const XT *__restrict__ src, bool ok, uint32_t h[4]);

// 8 consecutive binary16 values
template <>
__device__ __forceinline__ void load_x_piece<_Float16>(const _Float16 *__restrict__ src, bool ok,
                                                       uint32_t h[4]) {
    if (ok) {
        const u4_t v = *reinterpret_cast<const u4_t *>(src);
        h[0] = v[0]; h[1] = v[1]; h[2] = v[2]; h[3] = v[3];
    } else {
        h[0] = h[1] = h[2] = h[3] = 0u;
    }
}

// 8 consecutive float32 values rounded to binary16
template <>
__device__ __forceinline__ void load_x_piece<float>(const float *__restrict__ src, bool ok,
                                                    uint32_t h[4]) {
    if (ok) {
        const float4 a = *reinterpret_cast<const float4 *>(src);
        const float4 b = *reinterpret_cast<const float4 *>(src + 4);
        h[0] = as_u32(h2_t{(_Float16)a.x, (_Float16)a.y});
        h[1] = as_u32(h2_t{(_Float16)a.z, (_Float16)a.w});
        h[2] = as_u32(h2_t{(_Float16)b.x, (_Float16)b.y});
        h[3] = as_u32(h2_t{(_Float16)b.z, (_Float16)b.w});
    } else {
        h[0] = h[1] = h[2] = h[3] = 0u;
    }
}

template <typename XT>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_kernel(
    const uint8_t *__restrict__ packed, const XT *__restrict__ x, float *__restrict__ y,
    int64_t n, int64_t out, int64_t in) {
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][kGemmBM * kXRowBytes];
    const Layout L(out, in);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const Magic mg = pinned_magic();
    const int g = lane >> 4, r = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * kGemmBM;
    const int64_t tile0 = (int64_t)blockIdx.x * (kGemmBN / kTileRows) + wave * kGemmTilesPerWave;
    const int64_t nsteps = L.g4;

    // ---- staging of x: 64 rows x 16 pieces of 8 values per step -----------
    // piece p of a row covers k = 8p..8p+7 of the step: block s = p/4, offset
    // o = 8*(p%4) in the block.  Its first 4 values go to quarter
    // g = 2*((p%4)&1) (o = 0 or 16 -> g 0; o = 8 or 24 -> g 2) and the next
    // 4 to g + 1; o < 16 fills the first half of the 16-byte fragment,
    // o >= 16 the second half.
    uint32_t xh[4][4];
    auto load_x_step = [&](int64_t step) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + q * 256;
            const int row = c >> 4, p = c & 15;
            const int64_t tok = m0 + row;
            const int64_t k = step * 128 + 8 * p;
            const bool ok = tok < n && k < in;
            load_x_piece<XT>(x + tok * in + k, ok, xh[q]);
        }
    };
    auto store_x_step = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = tid + q * 256;
            const int row = c >> 4, p = c & 15;
            const int s = p >> 2, pq = p & 3;
            const int ga = (pq & 1) * 2, half = pq >> 1;
            uint8_t *base = xs[buf] + row * kXRowBytes + s * 64 + half * 8;
            *reinterpret_cast<u2_t *>(base + ga * 16) = u2_t{xh[q][0], xh[q][1]};
            *reinterpret_cast<u2_t *>(base + (ga + 1) * 16) = u2_t{xh[q][2], xh[q][3]};
        }
    };

    // ---- weight words: 4 tiles x (16-byte codes + 8-byte scales) per step --
    u4_t cw[kGemmTilesPerWave], cwn[kGemmTilesPerWave];
    u2_t sw[kGemmTilesPerWave], swn[kGemmTilesPerWave];
    auto load_w_step = [&](int64_t step, u4_t (&c)[kGemmTilesPerWave],
                           u2_t (&sc)[kGemmTilesPerWave]) {
#pragma unroll
        for (int ni = 0; ni < kGemmTilesPerWave; ++ni) {
            const int64_t t = tile0 + ni;
            if (t < L.tiles) {
                c[ni] = load_u4(packed + L.tile_codes(t) + step * kGroupCodeBytes + lane * 16);
                sc[ni] = load_u2(packed + L.tile_scales(t) + step * kGroupScaleBytes + r * 8);
            } else {
                c[ni] = u4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                sc[ni] = u2_t{0u, 0u};
            }
        }
    };

    f4_t acc[kGemmMSub][kGemmTilesPerWave];
#pragma unroll
    for (int mi = 0; mi < kGemmMSub; ++mi)
#pragma unroll
        for (int ni = 0; ni < kGemmTilesPerWave; ++ni) acc[mi][ni] = f4_t{0.f, 0.f, 0.f, 0.f};

    load_x_step(0);
    load_w_step(0, cw, sw);
    store_x_step(0);
    __syncthreads();

    int buf = 0;
    for (int64_t step = 0; step < nsteps; ++step) {
        const bool more = step + 1 < nsteps;
        if (more) {
            load_x_step(step + 1);
            load_w_step(step + 1, cwn, swn);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            h8_t a[kGemmMSub];
#pragma unroll
            for (int mi = 0; mi < kGemmMSub; ++mi) {
                const uint8_t *p = xs[buf] + (mi * 16 + r) * kXRowBytes + s * 64 + g * 16;
                a[mi] = __builtin_bit_cast(h8_t, *reinterpret_cast<const u4_t *>(p));
            }
#pragma unroll
            for (int ni = 0; ni < kGemmTilesPerWave; ++ni) {
                uint32_t q[4];
                decode_word(cw[ni][s], mg, q);
                const uint32_t dbits = (sw[ni][s >> 1] >> (16 * (s & 1))) & 0xFFFFu;
                const h2_t d2 = as_h2(dbits | (dbits << 16));
#pragma unroll
                for (int k = 0; k < 4; ++k) q[k] = as_u32(as_h2(q[k]) * d2);
                const h8_t bfrag = pack_h8(q);
#pragma unroll
                for (int mi = 0; mi < kGemmMSub; ++mi)
                    acc[mi][ni] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mi], bfrag, acc[mi][ni], 0, 0, 0);
            }
        }
        if (more) {
            store_x_step(buf ^ 1);
#pragma unroll
            for (int ni = 0; ni < kGemmTilesPerWave; ++ni) { cw[ni] = cwn[ni]; sw[ni] = swn[ni]; }
        }
        __syncthreads();
        buf ^= 1;
    }

    // ---- epilogue: D slot 4g+i of M sub-tile mi, weight row r of tile ni ---
#pragma unroll
    for (int mi = 0; mi < kGemmMSub; ++mi)
#pragma unroll
        for (int ni = 0; ni < kGemmTilesPerWave; ++ni) {
            const int64_t row = (tile0 + ni) * kTileRows + r;
            if (row >= out) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = m0 + mi * 16 + 4 * g + i;
                if (tok < n) y[tok * out + row] = acc[mi][ni][i];
            }
        }
}

bool gemm_supports(int64_t n, int64_t out, int64_t in, int x_f16) {
    (void)x_f16;
    const int64_t gy = (n + kGemmBM - 1) / kGemmBM;
    const int64_t gx = (out + kGemmBN - 1) / kGemmBN;
    return n >= 1 && out >= 1 && in >= 32 && gy <= 65535 && gx <= 0x7fffffff;
}

hipError_t launch_gemm(const void *packed, const void *x, int x_f16, float *y, int64_t n,
                       int64_t out, int64_t in, hipStream_t stream) {
    const dim3 grid((unsigned)((out + kGemmBN - 1) / kGemmBN), (unsigned)((n + kGemmBM - 1) / kGemmBM));
    const dim3 block(kGemmWaves * 64);
    if (x_f16)
        hipLaunchKernelGGL(gemm_kernel<_Float16>, grid, block, 0, stream, (const uint8_t *)packed,
                           (const _Float16 *)x, y, n, out, in);
    else
        hipLaunchKernelGGL(gemm_kernel<float>, grid, block, 0, stream, (const uint8_t *)packed,
                           (const float *)x, y, n, out, in);
    return hipGetLastError();
}

}  // namespace q4
