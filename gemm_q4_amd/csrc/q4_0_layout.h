// Repacked Q4_0 layout shared by the repack kernels and the matmul kernels.
//
// The matrix is cut into tiles of 16 consecutive rows, and each row's nb =
// in/32 blocks into groups of four consecutive blocks.  Rows are padded to a
// multiple of 16 and blocks to a multiple of 4 with zero blocks (scale +0,
// every code 8), so every tile holds 16 rows of g4 = ceil(nb/4) whole groups.
// Two streams:
//
//   scales : tiles * g4 * 128 bytes, at the start of the buffer.
//     tile t, group j, row r, block s of the group (b = 4j + s):
//         t*g4*128 + j*128 + r*8 + s*2                 (binary16 d)
//   codes  : tiles * g4 * 1024 bytes, after the scales.
//     tile t, group j, row r, quarter g (code bytes 4g..4g+3), block s:
//         t*g4*1024 + j*1024 + (g*16 + r)*16 + s*4     (4 bytes)
//
// So a wavefront lane l = g*16 + r reads one 16-byte word per (tile, group):
// the code bytes 4g..4g+3 of row r for the group's four blocks, and 8 bytes of
// scales (row r's four d).  The 64 lanes of a wave cover one contiguous 1 KB
// chunk.  Inside a block the split-half order is kept, so the word for quarter
// g holds weights 4g..4g+3 (low nibbles of its bytes) and 4g+16..4g+19 (high
// nibbles): exactly the eight K-values that lane l feeds a 16x16x32 MFMA when
// the tile's rows are the MFMA's N index.
#pragma once

#include <stdint.h>

namespace q4 {

constexpr int kTileRows = 16;
constexpr int kBlockK = 32;
constexpr int kGroupBlocks = 4;
constexpr int kGroupCodeBytes = 1024;
constexpr int kGroupScaleBytes = 128;

struct Layout {
    int64_t out, in, nb, tiles, g4;

    __host__ __device__ Layout(int64_t out_, int64_t in_)
        : out(out_), in(in_), nb(in_ / kBlockK),
          tiles((out_ + kTileRows - 1) / kTileRows),
          g4((in_ / kBlockK + kGroupBlocks - 1) / kGroupBlocks) {}

    __host__ __device__ int64_t scale_bytes() const { return tiles * g4 * kGroupScaleBytes; }
    __host__ __device__ int64_t total_bytes() const {
        return tiles * g4 * (kGroupScaleBytes + kGroupCodeBytes);
    }
    // Start of tile t's scale stream / code stream.
    __host__ __device__ int64_t tile_scales(int64_t t) const { return t * g4 * kGroupScaleBytes; }
    __host__ __device__ int64_t tile_codes(int64_t t) const {
        return scale_bytes() + t * g4 * kGroupCodeBytes;
    }
    // Byte offset of the scale of (tile t, row r, block b).
    __host__ __device__ int64_t scale_off(int64_t t, int r, int64_t b) const {
        return tile_scales(t) + (b >> 2) * kGroupScaleBytes + r * 8 + (b & 3) * 2;
    }
    // Byte offset of the 4 code bytes 4g..4g+3 of (tile t, row r, block b).
    __host__ __device__ int64_t code_off(int64_t t, int r, int g, int64_t b) const {
        return tile_codes(t) + (b >> 2) * kGroupCodeBytes + (g * 16 + r) * 16 + (b & 3) * 4;
    }
};

}  // namespace q4
