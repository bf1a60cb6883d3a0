// combine.hip -- gate-weighted combine back to token order.
//
// out[t] = sum_{j = 0 .. k-1} w[t][j] * Y[slot(t, j)] + sum_{s < S} Y[T*k + s*T + t],
// in fp32, j then s ascending (the shared experts, weight 1, after the routed
// sum), then rounded to the output type: the Hadamard-weighted combine of
// the FlashMoE Kernel page (Architecture, unified task abstraction), written
// back through the per-slot source record (MegaMoE-vs-MoE-systems page,
// section 2.4).  Each output element has exactly one writer, so there are no
// floating-point atomics and the result is bitwise reproducible.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// One workgroup per token row; each thread owns 8 consecutive columns (two
// 16-byte pieces) per pass, so d must be a multiple of 8 (the forward's shape
// rule already asks for 32).  The launch sizes the workgroup to d/8 lanes
// (up to 1024), so rows up to 8192 wide take one pass with no idle tail.
// The output is stored non-temporally: this layer never reads it back
// (measured: FP8 prefill combine 1.50 -> 1.44 ms; the same hint on the Y
// loads made it slower).  The slots are read in groups of up to 8 whose
// loads are all issued before their fmas, so more Y bytes are in flight per
// CU; the accumulation itself stays j ascending, then the shared experts.
constexpr int kCombineGroup = 8;

// Y rows are fp32, bf16 (MXFP4 layers) or fp16 codes with an exponent byte
// per 32 columns (bf16 and FP8 layers); every term is widened to fp32 (code
// * 2^x is exact) before its fma.
template <bool OUT_BF16, int YF>
__global__ __launch_bounds__(1024) void combine_kernel(const void* __restrict__ Yv,
                                                      const uint8_t* __restrict__ ye,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ token_slot,
                                                      void* __restrict__ out, int T, int d, int k,
                                                      int S) {
  const int t = blockIdx.x;
  __shared__ int32_t s_slot[1024 + 8];
  __shared__ float s_w[1024 + 8];
  const int n = k + S;  // terms: k routed (weight w), then S shared (weight 1)
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    if (j < k) {
      s_slot[j] = token_slot[static_cast<size_t>(t) * k + j];
      s_w[j] = w[static_cast<size_t>(t) * k + j];
    } else {
      s_slot[j] = static_cast<int32_t>(static_cast<int64_t>(T) * k +
                                       static_cast<int64_t>(j - k) * T + t);
      s_w[j] = 1.0f;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n; j0 += kCombineGroup) {
      f32x4 y0[kCombineGroup], y1[kCombineGroup];
#pragma unroll
      for (int u = 0; u < kCombineGroup; ++u) {
        if (j0 + u < n) {
          const size_t o = static_cast<size_t>(s_slot[j0 + u]) * d + c;
          if constexpr (YF == kYBF16) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Yv) + o);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              y0[u][2 * q] = __uint_as_float(raw[q] << 16);
              y0[u][2 * q + 1] = __uint_as_float(raw[q] & 0xffff0000u);
              y1[u][2 * q] = __uint_as_float(raw[2 + q] << 16);
              y1[u][2 * q + 1] = __uint_as_float(raw[2 + q] & 0xffff0000u);
            }
          } else if constexpr (YF == kYF16E) {
            typedef _Float16 h8 __attribute__((ext_vector_type(8)));
            const h8 raw = *reinterpret_cast<const h8*>(static_cast<const uint16_t*>(Yv) + o);
            // the 8 columns lie in one 32-column group (c is a multiple of 8)
            const float sc = exp2_int(static_cast<int>(ye[o / 32]) - 127);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              y0[u][q] = static_cast<float>(raw[q]) * sc;
              y1[u][q] = static_cast<float>(raw[4 + q]) * sc;
            }
          } else {
            const float* row = static_cast<const float*>(Yv) + o;
            y0[u] = *reinterpret_cast<const f32x4*>(row);
            y1[u] = *reinterpret_cast<const f32x4*>(row + 4);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCombineGroup; ++u) {
        if (j0 + u < n) {
          const int j = j0 + u;
          if (j < k) {
            const float g = s_w[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              a0[r] = __builtin_fmaf(g, y0[u][r], a0[r]);
              a1[r] = __builtin_fmaf(g, y1[u][r], a1[r]);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              a0[r] += y0[u][r];
              a1[r] += y1[u][r];
            }
          }
        }
      }
    }
    if (OUT_BF16) {
      uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(t) * d + c;
      auto pk = [](float lo, float hi) {
        return f32x2_to_bf16x2_rne(lo, hi);
      };
      __builtin_nontemporal_store(
          u32x4{pk(a0[0], a0[1]), pk(a0[2], a0[3]), pk(a1[0], a1[1]), pk(a1[2], a1[3])},
          reinterpret_cast<u32x4*>(o));
    } else {
      float* o = static_cast<float*>(out) + static_cast<size_t>(t) * d + c;
      __builtin_nontemporal_store(a0, reinterpret_cast<f32x4*>(o));
      __builtin_nontemporal_store(a1, reinterpret_cast<f32x4*>(o + 4));
    }
  }
}

}  // namespace

void launch_combine(const void* Y, int y_format, const uint8_t* ye, const float* w,
                    const int32_t* token_slot, void* out, int T, int d, int k, int S,
                    bool out_bf16, hipStream_t s) {
  if (T <= 0) return;
  const int threads = std::min(1024, std::max(64, (d / 8 + 63) / 64 * 64));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(T), dim3(threads), 0, s, Y, ye, w, token_slot, out, T, d, k, S);
  };
  if (out_bf16) {
    if (y_format == kYF16E) go(combine_kernel<true, kYF16E>);
    else if (y_format == kYBF16) go(combine_kernel<true, kYBF16>);
    else go(combine_kernel<true, kYF32>);
  } else {
    if (y_format == kYF16E) go(combine_kernel<false, kYF16E>);
    else if (y_format == kYBF16) go(combine_kernel<false, kYBF16>);
    else go(combine_kernel<false, kYF32>);
  }
}

}  // namespace moe
