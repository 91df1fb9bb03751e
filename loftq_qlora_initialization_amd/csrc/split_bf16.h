// Splitting fp32 values into two bf16 pieces for the bf16 matrix cores:
// hi = bf16(x), lo = bf16(x - hi), both rounded to nearest even.  x - hi is exact
// in fp32, and |x - hi - lo| <= 2^-18 |x|.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loftq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// hi/lo pieces of eight values, a pair at a time: one packed conversion for the
// two hi, their fp32 values back by a shift and a mask, two subtractions, one
// packed conversion for the two lo.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  u32x4v h, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * p], x[2 * p + 1]}, bf16x2));
    const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xFFFF0000u);
    h[p] = hp;
    l[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * p] - h0, x[2 * p + 1] - h1}, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}
__device__ __forceinline__ void split8(const float4& a, const float4& b, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  split8(x, hi, lo);
}
// N values (N even) as N / 2 packed words of hi and of lo pieces
template <int N>
__device__ __forceinline__ void split_pairs(const float (&x)[N], uint32_t (&h)[N / 2], uint32_t (&l)[N / 2]) {
#pragma unroll
  for (int p = 0; p < N / 2; ++p) {
    const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * p], x[2 * p + 1]}, bf16x2));
    const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xFFFF0000u);
    h[p] = hp;
    l[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * p] - h0, x[2 * p + 1] - h1}, bf16x2));
  }
}
__device__ __forceinline__ void split8_u4(const float (&x)[8], uint4& hi, uint4& lo) {
  bf16x8 h, l;
  split8(x, h, l);
  hi = __builtin_bit_cast(uint4, h);
  lo = __builtin_bit_cast(uint4, l);
}

}  // namespace
}  // namespace loftq
