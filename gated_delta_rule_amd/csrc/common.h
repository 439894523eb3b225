// Device helpers shared by the gfx950 kernels of libgdr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 -> fp32 on raw bits (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even with the hardware conversion (gfx950's packed
// f32 -> bf16 convert: identical to integer round-to-nearest-even on every
// non-NaN input, checked over all 2^32 bit patterns; a NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two values rounded as above, packed low = a, high = b (one instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t h;
  h[0] = (__bf16)a;
  h[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, h);
}

// Split x into bf16 hi + lo with hi = rne(x), lo = rne(x - hi): hi + lo
// carries about 16 significant bits of x.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_from_f32(T* p, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// Log-decays below this are taken as this: e^{-120} is zero in fp32 (and
// e^{g} for g < -120 is below 1e-52 in any format), so the state is reset
// exactly as the recurrence would; bounding g keeps the chunk-local
// cumulative sums and their differences finite (g = -inf would give
// -inf - -inf) and accurate.
constexpr float kMinLogDecay = -120.f;

// Reinterpret 8 raw bf16 words as the MFMA operand vector.
__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(16x32) * B(32x16) + C, bf16 operands, fp32 accumulate.
// Lane l holds A[m = l%16][k = 8*(l/16) + j], B[k = 8*(l/16) + j][n = l%16]
// (j = 0..7) and D[m = 4*(l/16) + i][n = l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum over the lanes of an aligned group of `width` lanes (power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum over the 8-lane group (lanes 8m .. 8m+7) with data-parallel-primitive
// moves (no LDS traffic); every lane gets the same value, since each step
// adds a lane pair in both orders.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_move<0x141>(x);  // row_half_mirror: lane i <-> 7 - i of its 8
  return x;
}

}  // namespace gdr
