// quant.hip -- FP8 1x128 group quantisation of the bf16 activations.
//
// Per group of 128 consecutive elements of a row: amax, scale s = amax / 448
// (1 when amax == 0) and codes e4m3_rne_sat(v / s), both quotients IEEE fp32
// -- the activation format the FP8 layer feeds its expert GEMMs (the
// activation + scale-factor load role on the MegaMoE-vs-MoE-systems page,
// section 2.1, consumes exactly these codes and scales).
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// 16 lanes per group (8 elements each), 4 groups per wavefront, 16 per block.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x,
                                                        int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int64_t s_stride) {
  const int64_t groups_per_row = cols / 128;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool valid = gid < rows * groups_per_row;
  const int64_t row = valid ? gid / groups_per_row : 0;
  const int64_t grp = valid ? gid - row * groups_per_row : 0;
  const int64_t base = row * cols + grp * 128 + sub * 8;
  float v[8];
  float m = 0.f;
  if (valid) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
  if (!valid) return;
  const float sc = (m == 0.f) ? 1.0f : __fdiv_rn(m, 448.0f);
  uint2 out;
  out.x = 0;
  out.y = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) out.x |= f32_to_e4m3(__fdiv_rn(v[i], sc)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) out.y |= f32_to_e4m3(__fdiv_rn(v[4 + i], sc)) << (8 * i);
  *reinterpret_cast<uint2*>(q + base) = out;
  if (sub == 0) s[row * s_stride + grp] = sc;
}

// OCP MX FP8 of the bf16 activations: blocks of 32 consecutive elements of a
// row share one E8M0 scale 2^X, X = floor(log2(amax)) - 8 (0 for an all-zero
// block), and each element becomes e4m3_rne_sat(v * 2^-X) -- the FP8
// activations of the FP8 x FP4 expert variant (MegaMoE-vs-MoE-systems page,
// section 1).  4 lanes per block (8 elements each), 64 blocks per workgroup.
__global__ __launch_bounds__(256) void quant_mx_kernel(const uint16_t* __restrict__ x,
                                                       int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ s) {
  const int64_t blocks_per_row = cols / 32;
  const int64_t bid = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool valid = bid < rows * blocks_per_row;
  const int64_t base = (valid ? bid : 0) * 32 + sub * 8;  // rows are contiguous
  float v[8];
  float m = 0.f;
  if (valid) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  if (!valid) return;
  const int e = mx_exponent_e4m3(m);
  uint2 out;
  out.x = 0;
  out.y = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) out.x |= f32_to_e4m3(__builtin_ldexpf(v[i], -e)) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) out.y |= f32_to_e4m3(__builtin_ldexpf(v[4 + i], -e)) << (8 * i);
  *reinterpret_cast<uint2*>(q + base) = out;
  if (sub == 0) s[bid] = static_cast<uint8_t>(e + 127);
}

}  // namespace

void launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                     hipStream_t st) {
  const int64_t blocks = rows * (cols / 32);
  if (blocks <= 0) return;
  quant_mx_kernel<<<dim3(static_cast<unsigned>((blocks + 63) / 64)), 256, 0, st>>>(x, rows, cols,
                                                                                    q, s);
}

void launch_quant_fp8(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* s,
                      int64_t s_stride, hipStream_t st) {
  const int64_t groups = rows * (cols / 128);
  if (groups <= 0) return;
  const int64_t blocks = (groups + 15) / 16;
  quant_fp8_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, st>>>(x, rows, cols, q, s,
                                                                        s_stride);
}

}  // namespace moe
