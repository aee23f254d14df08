// Device-side helpers for the Q4_0 kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_0_layout.h"

namespace q4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// Binary16 magic numbers: a 4-bit code q placed in the low mantissa bits of
// 0x6400 (2^10) reads as 1024 + q; placed four bits higher under 0x5400 (2^6)
// it reads as 64 + q.  Subtracting 1032 or 72 leaves q - 8 exactly.
constexpr uint32_t kMagicLo = 0x64006400u;
constexpr uint32_t kMagicHi = 0x54005400u;
constexpr uint32_t kMaskLo = 0x000F000Fu;
constexpr uint32_t kMaskHi = 0x00F000F0u;

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// The two magic words, held in vector registers.  gfx950's three-operand
// (VOP3) encoding takes no literal and at most one scalar operand, so with both
// the nibble mask and the magic as constants the compiler splits the masked
// insert into an AND and an OR.  An identity quad-permutation move hides the
// magic's value from constant folding; the insert then becomes one
// v_and_or_b32 (mask from a scalar register, magic from this vector register).
struct Magic {
    uint32_t lo, hi;
};
__device__ __forceinline__ Magic pinned_magic() {
    Magic m;
    m.lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)kMagicLo, 0xE4, 0xF, 0xF, true);
    m.hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)kMagicHi, 0xE4, 0xF, 0xF, true);
    return m;
}

// Decode one 4-byte code word (code bytes 4g..4g+3 of a block) into the eight
// exact values q - 8 as binary16, in the order
//   k = 4g+0, 4g+1, 4g+2, 4g+3, 4g+16, 4g+17, 4g+18, 4g+19.
// Byte i carries weight 4g+i in its low nibble and 4g+16+i in its high
// nibble (split-half order).  v_perm spreads bytes 0,1 (then 2,3) into the
// two 16-bit halves; one masked insert per pair puts the nibbles under the
// magic exponents; one v_pk_add_f16 per pair removes the offset.
__device__ __forceinline__ void decode_word(uint32_t w, const Magic &m, uint32_t q[4]) {
    const uint32_t t01 = __builtin_amdgcn_perm(w, w, 0x0C010C00u);  // B0,0,B1,0
    const uint32_t t23 = __builtin_amdgcn_perm(w, w, 0x0C030C02u);  // B2,0,B3,0
    const h2_t off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    q[0] = as_u32(as_h2((t01 & kMaskLo) | m.lo) + off_lo);
    q[1] = as_u32(as_h2((t23 & kMaskLo) | m.lo) + off_lo);
    q[2] = as_u32(as_h2((t01 & kMaskHi) | m.hi) + off_hi);
    q[3] = as_u32(as_h2((t23 & kMaskHi) | m.hi) + off_hi);
}

// Same eight values in a cheaper order (one shift, no v_perm):
//   k = 4g+0, 4g+2, 4g+16, 4g+18, 4g+1, 4g+3, 4g+17, 4g+19.
// Used where the consumer lays its activation operands out to match.
__device__ __forceinline__ void decode_word_pairs(uint32_t w, const Magic &m, uint32_t q[4]) {
    const uint32_t w8 = w >> 8;
    const h2_t off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    q[0] = as_u32(as_h2((w & kMaskLo) | m.lo) + off_lo);
    q[1] = as_u32(as_h2((w & kMaskHi) | m.hi) + off_hi);
    q[2] = as_u32(as_h2((w8 & kMaskLo) | m.lo) + off_lo);
    q[3] = as_u32(as_h2((w8 & kMaskHi) | m.hi) + off_hi);
}

__device__ __forceinline__ h8_t pack_h8(const uint32_t q[4]) {
    u4_t u = {q[0], q[1], q[2], q[3]};
    return __builtin_bit_cast(h8_t, u);
}

__device__ __forceinline__ u4_t load_u4(const uint8_t *p) {
    return *reinterpret_cast<const u4_t *>(p);
}
__device__ __forceinline__ u2_t load_u2(const uint8_t *p) {
    return *reinterpret_cast<const u2_t *>(p);
}
__device__ __forceinline__ uint32_t load_u32(const uint8_t *p) {
    return *reinterpret_cast<const uint32_t *>(p);
}
__device__ __forceinline__ uint32_t load_u16(const uint8_t *p) {
    return *reinterpret_cast<const uint16_t *>(p);
}

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }

}  // namespace q4
