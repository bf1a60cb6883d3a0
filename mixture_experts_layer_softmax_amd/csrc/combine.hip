// combine.hip -- gate-weighted combine back to token order.
//
// out[t] = sum_{j = 0 .. k-1} w[t][j] * Y[slot(t, j)] + sum_{s < S} Y[T*k + s*T + t],
// in fp32, j then s ascending (the shared experts, weight 1, after the routed
// sum), then rounded to the output type: the Hadamard-weighted combine of
// the FlashMoE Kernel page (Architecture, unified task abstraction), written
// back through the per-slot source record (MegaMoE-vs-MoE-systems page,
// section 2.4).  Each output element has exactly one writer, so there are no
// floating-point atomics and the result is bitwise reproducible.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// One workgroup per token row; each thread owns 4 consecutive columns.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ token_slot,
                                                      void* __restrict__ out, int T, int d, int k,
                                                      int S) {
  const int t = blockIdx.x;
  __shared__ int32_t s_slot[1024];
  __shared__ float s_w[1024];
  for (int j = threadIdx.x; j < k; j += 256) {
    s_slot[j] = token_slot[static_cast<size_t>(t) * k + j];
    s_w[j] = w[static_cast<size_t>(t) * k + j];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(Y + static_cast<size_t>(s_slot[j]) * d + c);
      const float g = s_w[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(g, y[r], acc[r]);
    }
    for (int sh = 0; sh < S; ++sh) {
      const size_t slot = static_cast<size_t>(T) * k + static_cast<size_t>(sh) * T + t;
      const f32x4 y = *reinterpret_cast<const f32x4*>(Y + slot * d + c);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += y[r];
    }
    if (OUT_BF16) {
      uint2 v;
      v.x = f32_to_bf16_rne(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[1])) << 16);
      v.y = f32_to_bf16_rne(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + static_cast<size_t>(t) * d + c) = v;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + static_cast<size_t>(t) * d + c) = acc;
    }
  }
}

}  // namespace

void launch_combine(const float* Y, const float* w, const int32_t* token_slot, void* out,
                    int T, int d, int k, int S, bool out_bf16, hipStream_t s) {
  if (T <= 0) return;
  if (out_bf16)
    combine_kernel<true><<<T, 256, 0, s>>>(Y, w, token_slot, out, T, d, k, S);
  else
    combine_kernel<false><<<T, 256, 0, s>>>(Y, w, token_slot, out, T, d, k, S);
}

}  // namespace moe
