// Shared device-side definitions for the gfx950 kernels of libckl.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckl {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kIdxEnd = 0x7fffffff;  // sentinel past every vocabulary index

// bf16 <-> f32.  Widening is exact; narrowing rounds to nearest, ties to
// even: the language conversion, which gfx950 executes as one
// v_cvt_pk_bf16_f32 per pair of values.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(bf16_t)lo, (bf16_t)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)f);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// The value itself, opaque to the optimizer: a cheap expression derived from
// it inside a loop is computed there instead of being hoisted out and held in
// a register across the loop (where it would crowd out the accumulators).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge two online log-sum-exp states kept in base-2 units: (m, s) stands for
// log2(s) + m = log2 sum 2^x over the elements seen.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) { m = mn; s = 0.f; return; }
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

}  // namespace ckl
