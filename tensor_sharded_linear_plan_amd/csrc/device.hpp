// Device-side helpers shared by the gfx950 kernels: vector types, number
// format conversions and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- number formats -------------------------------------------------------

// bf16 bit pattern -> binary32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two binary32 values -> packed bf16 pair, round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// ---- 4-bit codes ------------------------------------------------------------
// A packed code word holds eight consecutive k of one column: even k in the
// low half-word (nibbles 0..3), odd k in the high half-word (nibbles 4..7),
// so (w >> 4j) & 0x000F000F isolates the pair (k = 2j, 2j + 1).

// Word -> four bf16 pairs holding 128 + q (0x4300 is bf16 128.0 and its 7
// mantissa bits count units of 1 there).  gfx9 VOP3 encodings take no
// literal operand and at most one scalar one, so with the two constants
// visible the compiler spends a separate AND and OR per pair; loaded
// opaquely (the mask into a vector register, the other into a scalar one)
// they let it select one v_and_or_b32 per pair.
__device__ __forceinline__ bf16x8 q4_to_bf16_plus128(uint32_t w) {
    uint32_t m, o;
    asm("v_mov_b32 %0, 0x000f000f" : "=v"(m));
    asm("s_mov_b32 %0, 0x43004300" : "=s"(o));
    u32x4 r;
    r.x = (w & m) | o;
    r.y = ((w >> 4) & m) | o;
    r.z = ((w >> 8) & m) | o;
    r.w = ((w >> 12) & m) | o;
    return __builtin_bit_cast(bf16x8, r);
}

// ---- MFMA ---------------------------------------------------------------------
// 16x16 output tile per wave.  Operand lane layout (as used by every kernel
// here): lane l feeds row (A) / column (B) l % 16 with a run of k values
// selected by l / 16; both operands use the same k run, which is all a dot
// product needs.  Accumulator: lane l holds rows 4 * (l / 16) + i, i < 4,
// of column l % 16.

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

} // namespace tsl
