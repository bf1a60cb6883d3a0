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

// One workgroup per token row; each thread owns kSlotBytes of a Y row per
// pass (CPT columns: 8 fp32 or 16 two-byte ones), so d must be a multiple of
// 16 (the forward's shape rule already asks for 32).  The launch sizes the
// workgroup to d/CPT lanes (up to 1024).  The output is
// stored non-temporally: this layer never reads it back (measured: FP8
// prefill combine 1.50 -> 1.44 ms; the same hint on the Y loads made it
// slower).  The slots are read in groups of up to 8 whose loads are all
// issued before their fmas, so more Y bytes are in flight per CU; the
// accumulation itself stays j ascending, then the shared experts.
constexpr int kCombineGroup = 8;
constexpr int kSlotBytes = 32;

template <int YF>
constexpr int combine_cols() { return kSlotBytes / (YF == kYF32 ? 4 : 2); }

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
  constexpr int CPT = combine_cols<YF>();
  constexpr int NV = CPT / 4;             // f32x4 accumulators per thread
  constexpr int NP = kSlotBytes / 16;     // 16-byte pieces per slot
  static_assert(32 % CPT == 0, "a thread's fp16 columns lie in one 32-column group");
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
  for (int c = threadIdx.x * CPT; c < d; c += blockDim.x * CPT) {
    f32x4 a[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) a[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n; j0 += kCombineGroup) {
      // the group's 32 bytes per slot, as loaded (converted at the fma)
      u32x4 raw[kCombineGroup][NP];
      float sc[kCombineGroup];
#pragma unroll
      for (int u = 0; u < kCombineGroup; ++u) {
        sc[u] = 1.0f;
        if (j0 + u < n) {
          const size_t o = static_cast<size_t>(s_slot[j0 + u]) * d + c;
          const uint8_t* row = static_cast<const uint8_t*>(Yv) + o * (YF == kYF32 ? 4 : 2);
#pragma unroll
          for (int pc = 0; pc < NP; ++pc) raw[u][pc] = *reinterpret_cast<const u32x4*>(row + 16 * pc);
          // (fp16: the CPT columns lie in one 32-column group)
          if constexpr (YF == kYF16E) sc[u] = exp2_int(static_cast<int>(ye[o / 32]) - 127);
        }
      }
#pragma unroll
      for (int u = 0; u < kCombineGroup; ++u) {
        if (j0 + u < n) {
          const int j = j0 + u;
          const float g = s_w[j];
          float y[CPT];
#pragma unroll
          for (int q = 0; q < 4 * NP; ++q) {
            const uint32_t b = raw[u][q / 4][q % 4];
            if constexpr (YF == kYF32) {
              y[q] = __uint_as_float(b);
            } else if constexpr (YF == kYBF16) {
              y[2 * q] = __uint_as_float(b << 16);
              y[2 * q + 1] = __uint_as_float(b & 0xffff0000u);
            } else {
              typedef _Float16 h2 __attribute__((ext_vector_type(2)));
              const h2 hv = __builtin_bit_cast(h2, b);
              y[2 * q] = static_cast<float>(hv[0]) * sc[u];
              y[2 * q + 1] = static_cast<float>(hv[1]) * sc[u];
            }
          }
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              a[v][r] = (j < k) ? __builtin_fmaf(g, y[4 * v + r], a[v][r]) : a[v][r] + y[4 * v + r];
        }
      }
    }
    if constexpr (OUT_BF16) {
      uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(t) * d + c;
#pragma unroll
      for (int v = 0; v < NV; v += 2)
        __builtin_nontemporal_store(
            u32x4{f32x2_to_bf16x2_rne(a[v][0], a[v][1]), f32x2_to_bf16x2_rne(a[v][2], a[v][3]),
                  f32x2_to_bf16x2_rne(a[v + 1][0], a[v + 1][1]),
                  f32x2_to_bf16x2_rne(a[v + 1][2], a[v + 1][3])},
            reinterpret_cast<u32x4*>(o + 4 * v));
    } else {
      float* o = static_cast<float*>(out) + static_cast<size_t>(t) * d + c;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        __builtin_nontemporal_store(a[v], reinterpret_cast<f32x4*>(o + 4 * v));
    }
  }
}

}  // namespace

void launch_combine(const void* Y, int y_format, const uint8_t* ye, const float* w,
                    const int32_t* token_slot, void* out, int T, int d, int k, int S,
                    bool out_bf16, hipStream_t s) {
  if (T <= 0) return;
  const int cpt = y_format == kYF32 ? combine_cols<kYF32>() : combine_cols<kYF16E>();
  const int threads = std::min(1024, std::max(64, (d / cpt + 63) / 64 * 64));
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
