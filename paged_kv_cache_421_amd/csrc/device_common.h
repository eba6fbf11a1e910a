// Internal device helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pagedkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = PA_BLOCK_SIZE;
constexpr int kPartTokens = PA_PARTITION_TOKENS;
constexpr int kPartBlocks = kPartTokens / kBlock;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP E4M3 ("e4m3fn") encoder: round-to-nearest-even of y, saturating to
// +-448, NaN -> 0x7F, sign kept (so -0 and tiny negatives give 0x80).
// Built from the format's fields, independent of the hardware converter.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                 // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // |y| >= 448 (and inf)
  uint32_t mag;
  if (a < 0x3C800000u) {                             // |y| < 2^-6: subnormal step 2^-9
    // |y| * 512 is exact; rint is round-half-even; 8 lands on code 0x08 = 2^-6
    mag = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  } else {
    // keep 3 mantissa bits with round-half-even at bit 20, then move the
    // exponent bias from 127 to 7 (a carry out of the mantissa bumps the
    // exponent, which is the right result)
    mag = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return sign | mag;
}

// Publishing partial results to other waves: the stores are issued, then
// this waits until every memory access of the wave has completed, before the
// arrival counter is bumped.  The memory clobber keeps the compiler from
// moving any memory access across the wait (a relaxed atomic alone would let
// it schedule the counter update ahead of the stores).
__device__ __forceinline__ void wait_memory_done() {
  asm volatile("s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)" ::: "memory");
}

// Compiler-only barrier: memory accesses are not moved across it.  Placed
// after an arrival-counter update whose result decides whether the wave
// reads the other waves' results, so those loads stay after the update.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

}  // namespace pagedkv
