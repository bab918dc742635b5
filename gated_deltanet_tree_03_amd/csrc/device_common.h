// Device-side helpers for gfx950 (CDNA4): bf16 vector types, conversions,
// input loads for the two input dtypes, and 16-lane DPP reductions.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace treewy {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }

// Split x into hi + lo, both bf16: hi = bf16(x), lo = bf16(x - hi).  The
// residual x - hi - lo is below 2^-16 |x| (two 8-bit significands).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - static_cast<float>(hi));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// split_bf16 for a pair, as packed bf16 pairs (element 0 in the low half):
// one packed round-to-nearest-even conversion gives both hi values, whose
// fp32 values are two bit operations away; converted one by one, each hi
// value was rounded twice (once packed for the operand, once alone for the
// residual).
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
  const float r0 = x0 - __uint_as_float(h << 16);
  const float r1 = x1 - __uint_as_float(h & 0xffff0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

__device__ __forceinline__ void split_bf16x4(const float* x, bf16x4& hi, bf16x4& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) split_bf16x2(x[2 * p], x[2 * p + 1], h[p], l[p]);
  hi = __builtin_bit_cast(bf16x4, make_uint2(h[0], h[1]));
  lo = __builtin_bit_cast(bf16x4, make_uint2(l[0], l[1]));
}

__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) split_bf16x2(x[2 * p], x[2 * p + 1], h[p], l[p]);
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// Scalar input load for q/k/v/alpha/beta, bf16 bit patterns or fp32.
template <bool F32>
__device__ __forceinline__ float load_in(const void* base, int64_t idx) {
  if constexpr (F32) {
    return static_cast<const float*>(base)[idx];
  } else {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  }
}

// Four consecutive inputs starting at idx (idx % 4 == 0), widened to fp32.
template <bool F32>
__device__ __forceinline__ float4 load_in4(const void* base, int64_t idx) {
  if constexpr (F32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
}

// DPP cross-lane moves inside a 16-lane row (gfx9 DPP controls).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <-> 7-i within each half row
  x += dpp_mov<0x140>(x);  // row_mirror: lane i <-> 15-i
  return x;
}

__device__ __forceinline__ float qnan() { return __uint_as_float(0x7fc00000u); }

}  // namespace treewy
