// Helpers of the prefill kernel: direct copies from global memory into LDS
// and explicit waits on them.
#pragma once

#include "q4_0_device.h"

namespace q4 {

typedef float f16x_t __attribute__((ext_vector_type(16)));

// Direct copy of 16 bytes per lane from global memory into LDS (no register
// round trip): the wave's 64 lanes fill 1 KB at `lds` (wave-uniform), lane i
// at lds + 16 i.  Written as inline assembly on purpose: the compiler does not
// know which LDS bytes such a copy writes, so for its own copy instruction it
// waits for every outstanding copy before each later LDS read, which would
// drain the multi-stage pipeline below.  Here the copies are invisible to it
// and the kernel waits for them explicitly (vector-memory count, then a
// barrier) before reading a stage.  M0 holds the LDS base; one wait state
// separates its write from the copy.
__device__ __forceinline__ void dma16(const void *src, uint8_t *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(base)
                 : "memory", "m0");
}

// The same copy from a wave-uniform 64-bit base (scalar registers) plus a
// 32-bit byte offset per lane: offsets computed once stay in registers across
// a loop and only the base moves, so a copy costs no vector address
// arithmetic.
__device__ __forceinline__ void dma16_at(const void *base, uint32_t off, uint8_t *lds) {
    const uint32_t lb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lb)
                 : "memory", "m0");
}

static __device__ const u4_t kZeroPiece = {0u, 0u, 0u, 0u};

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt left
// free): vmcnt is bits 3:0 and 15:14 of the immediate.
#define Q4_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 0xF) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))
#define Q4_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

}  // namespace q4
