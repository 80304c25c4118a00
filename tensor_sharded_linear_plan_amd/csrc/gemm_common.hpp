// Device helpers shared by the GEMM kernels of the prefill regime: LDS
// sizing, the activation-block swizzle, direct global -> LDS copies and
// explicit wait counts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace tsl {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS a workgroup may use on gfx950.
constexpr int kLdsLimit = 160 * 1024;

// XOR swizzle of an activation row's 16-byte chunks in its LDS block, so
// that the 32 rows of a fragment read spread over all banks.
template <int CPR>
__device__ __forceinline__ int swz(int row_in_block) {
    return CPR == 8 ? (row_in_block & 7) : ((row_in_block >> 2) & 3);
}

// One wave instruction: lane l copies the 16 bytes at base + off (base
// wave-uniform, off a per-lane 32-bit byte offset) into LDS at lds + 16 l
// (lds wave-uniform).  Issued as inline assembly so that the compiler's
// wait-count tracking does not drain every outstanding copy before each LDS
// read; completion is awaited explicitly (vmcnt) before the barrier that
// publishes a stage.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}

// The same from a full 64-bit address per lane: 16 bytes (LDS at lds +
// 16 l) or 4 bytes (LDS at lds + 4 l).
__device__ __forceinline__ void dma16_at(const char *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(addr)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4_at(const char *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds), "v"(addr)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// s_waitcnt lgkmcnt(0) leaving the other counters alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }


} // namespace tsl
