// Internal helpers shared by the HIP kernels of libulysses (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uly {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte store, nontemporal, written through L2 at agent scope (sc1), for
// streams whose output is not read back soon (the swaps, the ring merge and
// gradient sum): no dirty lines are left in the XCD's L2 for later
// eviction. One line of inline assembly, since no builtin sets the scope
// bit; a store has no result, so the compiler's wait for the stored value
// stays in place.
__device__ __forceinline__ void store_through(void *p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(p), "v"(v) : "memory");
}

// Unsigned division of 32-bit values by a runtime divisor via a
// multiply-high and a shift (Granlund & Montgomery, "Division by Invariant
// Integers using Multiplication", PLDI 1994, round-up variant with a 33-bit
// magic held as 32 bits plus an add-and-shift step).
struct FastDiv {
  uint32_t div;
  uint32_t mul;
  uint32_t shift;

  __host__ __device__ FastDiv() : div(1), mul(0), shift(0) {}
  __host__ explicit FastDiv(uint32_t d) : div(d) {
    // l = ceil(log2(d)); m' = floor(2^32 * (2^l - d) / d) + 1
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    shift = l;
    uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    mul = (uint32_t)m;
  }
  __host__ __device__ __forceinline__ uint32_t q(uint32_t n) const {
    if (shift == 0) return n;  // div == 1
    uint32_t t = (uint32_t)(((uint64_t)n * mul) >> 32);
    return (t + ((n - t) >> 1)) >> (shift - 1);
  }
};

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32;
// `lo` lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace uly
