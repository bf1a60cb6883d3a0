// device_common.hpp -- small device helpers shared by the HIP kernels of
// libmoe.so (number-format conversions, wave reductions, vector types).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // 16-byte chunk
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448.
// Written from the format definition: 4 exponent bits (bias 7), 3 mantissa
// bits, subnormal spacing 2^-9, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(v);
  if (!(a < 448.0f)) return sign | 0x7eu;      // saturate (NaN not expected)
  if (a < 0.015625f) {                         // below 2^-6: multiples of 2^-9
    float m = __builtin_rintf(a * 512.0f);     // exact scaling, RNE
    return sign | static_cast<uint32_t>(m);    // m == 8 encodes 2^-6 exactly
  }
  uint32_t au = __float_as_uint(a);
  // re-bias the exponent from 127 to 7 and keep 3 mantissa bits with RNE;
  // a mantissa carry moves into the exponent field, which is what we want
  uint32_t biased = au - ((127u - 7u) << 23);
  uint32_t r = biased + 0x7ffffu + ((biased >> 20) & 1u);
  uint32_t code = r >> 20;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// Shared exponent X of an OCP MX block of E4M3 elements (scale 2^X, stored
// as the E8M0 byte X + 127): floor(log2(amax)) - 8, clamped below at -127
// (which also covers fp32 subnormal amax); 0 for an all-zero block.
__device__ __forceinline__ int mx_exponent_e4m3(float amax) {
  if (amax == 0.f) return 0;
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  return max(-127, e - 127 - 8);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace moe
