// Device-side helpers shared by the HIP kernels of libheadattn.so (vector
// types, buffer descriptors, half-wave exchanges, bf16 packing, the pivot
// thresholds of the online softmax).  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <utility>

#include "common.h"

namespace headattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) uint4 lds_uint4;
typedef __attribute__((address_space(3))) char lds_char;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// One bf16 row of K, V, Q or O (d = 64).
constexpr uint32_t kRowBytes = kHeadDim * 2;

// Word 3 of a raw buffer descriptor on the gfx9 family: 32-bit elements,
// no swizzle, range checked against word 2 (offsets past it read as zero and
// their writes are dropped).
constexpr uint32_t kBufferWord3 = 0x00020000u;
// A byte offset the range check always rejects.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Online-softmax pivot thresholds.  A pivot moves up when a tile's weights
// under it would pass 2^64, and down (only while a row has summed nothing)
// when they would fall below 2^-64: in fp32 that keeps every partial sum and
// every weighted V sum far from overflow and from the subnormal range.
// Kernels that compare sums use kPivotHigh / kPivotLow; those that compare
// log2-domain gaps (largest exponent minus pivot) use kPivotUp / kPivotDown.
constexpr float kPivotHigh = 0x1p64f;
constexpr float kPivotLow = 0x1p-64f;
constexpr float kPivotUp = 64.f;
constexpr float kPivotDown = -64.f;

// Lanes l and l ^ 32 of a 32x32 MFMA accumulator hold the same query row:
// combine the two half-waves with one v_permlane32_swap.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t a = r[0], b = r[1];
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ bool half_swap_or(bool x) {
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (r[0] | r[1]) != 0;
}

// Two floats rounded to nearest-even bf16 and packed, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Weights 2^x of one query block of a tile from its exponents x (key blocks
// x0: keys 0..31, x1: keys 32..63), packed to bf16 pairs in the order P.V
// consumes them.
__device__ __forceinline__ void exp_pack(const f32x16& x0, const f32x16& x1, uint32_t (&pk)[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pk[i] = pack_bf16x2(__builtin_amdgcn_exp2f(x0[2 * i]), __builtin_amdgcn_exp2f(x0[2 * i + 1]));
    pk[8 + i] = pack_bf16x2(__builtin_amdgcn_exp2f(x1[2 * i]), __builtin_amdgcn_exp2f(x1[2 * i + 1]));
  }
}

// Max of the 32 values of two accumulator blocks as a shallow tree of
// 3-input maxima.  The inputs are results of fp32 arithmetic (canonical), so
// each fmaxf pair folds into one v_max3_f32.
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = a[i];
    v[16 + i] = b[i];
  }
  float m[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) m[i] = fmaxf(fmaxf(v[3 * i], v[3 * i + 1]), v[3 * i + 2]);
  m[10] = fmaxf(v[30], v[31]);
  const float n0 = fmaxf(fmaxf(m[0], m[1]), m[2]);
  const float n1 = fmaxf(fmaxf(m[3], m[4]), m[5]);
  const float n2 = fmaxf(fmaxf(m[6], m[7]), m[8]);
  const float n3 = fmaxf(m[9], m[10]);
  return fmaxf(fmaxf(fmaxf(n0, n1), n2), n3);
}

__device__ __forceinline__ void barrier_lds() {
  // Block the compiler from moving memory accesses across, without the
  // vmcnt(0) a workgroup fence would add for the in-flight LDS fills; the
  // scheduling barriers keep register-only work (MFMAs on prefetched
  // fragments) in its phase as well.
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

}  // namespace headattn
