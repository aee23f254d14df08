// Repack kernels: GGUF Q4_0 blocks <-> the tiled two-stream layout of
// q4_0_layout.h.  Pure byte moves, so the round trip is bit exact.
#include "q4_0_internal.h"

namespace q4 {

// One thread per (tile, padded block, lane): lane l = g*16 + r moves code
// bytes 4g..4g+3 of row r, and lanes with g == 0 move the row's scale.
// Padding rows and padding blocks get scale +0 and codes 8 (weight 0).
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ src,
                                                     uint8_t *__restrict__ dst,
                                                     int64_t out, int64_t in) {
    const Layout L(out, in);
    const int64_t nbp = L.g4 * kGroupBlocks;
    const int64_t total = L.tiles * nbp * 64;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
         id += stride) {
    const int lane = (int)(id & 63);
    const int64_t b = (id >> 6) % nbp;
    const int64_t t = (id >> 6) / nbp;
    const int g = lane >> 4, r = lane & 15;
    const int64_t row = t * kTileRows + r;

    uint32_t word = 0x88888888u;   // padding: codes 8 -> weight 0
    uint32_t scale = 0;            // padding: scale +0
    if (row < out && b < L.nb) {
        const uint8_t *blk = src + (row * L.nb + b) * 18;
        word = (uint32_t)blk[2 + 4 * g] | ((uint32_t)blk[3 + 4 * g] << 8) |
               ((uint32_t)blk[4 + 4 * g] << 16) | ((uint32_t)blk[5 + 4 * g] << 24);
        scale = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
    }
    *reinterpret_cast<uint32_t *>(dst + L.code_off(t, r, g, b)) = word;
    if (g == 0)
        *reinterpret_cast<uint16_t *>(dst + L.scale_off(t, r, b)) = (uint16_t)scale;
    }
}

// One thread per (row < out, block, quarter g).
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ src,
                                                     uint8_t *__restrict__ dst,
                                                     int64_t out, int64_t in) {
    const Layout L(out, in);
    const int64_t total = out * L.nb * 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
         id += stride) {
    const int g = (int)(id & 3);
    const int64_t b = (id >> 2) % L.nb;
    const int64_t row = (id >> 2) / L.nb;
    const int64_t t = row / kTileRows;
    const int r = (int)(row % kTileRows);
    const uint32_t word = *reinterpret_cast<const uint32_t *>(src + L.code_off(t, r, g, b));
    uint8_t *blk = dst + (row * L.nb + b) * 18;
    blk[2 + 4 * g] = (uint8_t)(word & 0xFF);
    blk[3 + 4 * g] = (uint8_t)((word >> 8) & 0xFF);
    blk[4 + 4 * g] = (uint8_t)((word >> 16) & 0xFF);
    blk[5 + 4 * g] = (uint8_t)(word >> 24);
    if (g == 0) {
        const uint16_t s = *reinterpret_cast<const uint16_t *>(src + L.scale_off(t, r, b));
        blk[0] = (uint8_t)(s & 0xFF);
        blk[1] = (uint8_t)(s >> 8);
    }
    }
}

hipError_t launch_repack(const void *blocks, void *packed, int64_t out, int64_t in,
                         hipStream_t stream) {
    const Layout L(out, in);
    const int64_t total = L.tiles * L.g4 * kGroupBlocks * 64;
    const int64_t grid = grid_for(total, 256);
    hipLaunchKernelGGL(repack_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t *)blocks, (uint8_t *)packed, out, in);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *packed, void *blocks, int64_t out, int64_t in,
                         hipStream_t stream) {
    const Layout L(out, in);
    const int64_t total = out * L.nb * 4;
    const int64_t grid = grid_for(total, 256);
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t *)packed, (uint8_t *)blocks, out, in);
    return hipGetLastError();
}

}  // namespace q4
