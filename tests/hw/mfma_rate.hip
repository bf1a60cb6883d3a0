// Register-only MFMA issue rates of gfx950: what the matrix cores sustain
// with no memory traffic at all, for each MFMA form the library uses.
//
// One workgroup per CU (a 96 KB dynamic LDS request keeps a second one off
// the CU), W waves per SIMD, each wave running NACC independent accumulators
// through `iters` steps of one MFMA form whose operands never leave the
// registers.  Wave 0 of each workgroup reads the shader clock (s_memtime)
// and the 100 MHz reference clock (s_memrealtime) between two workgroup
// barriers around the loop.
// Output, one line per case:
//   case NAME waves_per_simd W chains N clk_per_mfma C flop_per_clk_cu F
//        mhz M tflops T pct_of_2400mhz_peak P
// clk_per_mfma is the SIMD's shader clocks per MFMA (all its waves
// together); the per-CU peaks at the nominal clock are 4096 (bf16), 8192
// (fp8 and fp4 forms) and 256 (fp32) FLOP per clock.  The dependent-chain
// cases (one wave per SIMD, one accumulator) give the issue-to-issue
// interval of back-to-back MFMAs that accumulate into the same registers,
// which bounds a sequential fp32 fma chain such as the gate's logits.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;

namespace {

enum Kind { kBF16 = 0, kFP8 = 1, kFP4xFP8 = 2, kFP4 = 3, kF32 = 4 };

constexpr int kLdsPad = 96 * 1024;  // one workgroup per CU

__host__ __device__ constexpr double flop_of(int kind) {
  return kind == kBF16 ? 2.0 * 16 * 16 * 32 : (kind == kF32 ? 2.0 * 16 * 16 * 4 : 2.0 * 16 * 16 * 128);
}

template <int KIND, int NACC>
__global__ void rate_kernel(float* out, int iters, unsigned long long* clk, int seed) {
  extern __shared__ uint8_t pad[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int s = lane + seed;
  // operands: varied, finite codes (E4M3 bytes with the top bit pattern 0x77
  // mask never form the NaN code 0x7f; every E2M1 nibble is a number)
  bf16x8 ab, bb;
  i32x8 a8, b8, a4, b4;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    ab[q] = static_cast<__bf16>(0.001f * static_cast<float>((s * 7 + q * 3) % 61 - 30));
    bb[q] = static_cast<__bf16>(0.002f * static_cast<float>((s * 5 + q * 11) % 53 - 26));
    const unsigned u = static_cast<unsigned>(s * 2654435761u + q * 40503u);
    a8[q] = static_cast<int>(u & 0x77777777u);
    b8[q] = static_cast<int>((u >> 3) & 0x77777777u);
    a4[q] = q < 4 ? static_cast<int>(u ^ 0x5a5a5a5au) : 0;
    b4[q] = q < 4 ? static_cast<int>(u * 3u) : 0;
  }
  const float af = 0.01f * static_cast<float>(s % 17), bf = 0.02f * static_cast<float>(s % 13);
  f32x4 acc[NACC];
#pragma unroll
  for (int c = 0; c < NACC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the barriers make the stamps span every wave of the workgroup: the
  // waves of one SIMD do not finish together (the older one wins the MFMA
  // arbitration), so one wave's own loop time would undercount the SIMD's
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < NACC; ++c) {
      if constexpr (KIND == kBF16)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, acc[c], 0, 0, 0);
      else if constexpr (KIND == kFP8)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[c], 0, 0, 0, 127,
                                                                  0, 127);
      else if constexpr (KIND == kFP4xFP8)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a4, b8, acc[c], 4, 0, 0, 127,
                                                                  0, 127);
      else if constexpr (KIND == kFP4)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a4, b4, acc[c], 4, 4, 0, 127,
                                                                  0, 127);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bf, acc[c], 0, 0, 0);
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < NACC; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[blockIdx.x * blockDim.x + tid] = sum;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (sum == 1234.5f) pad[tid] = 1;  // keeps the LDS request (never true in practice)
}

template <int KIND, int NACC>
int run(const char* name, int waves_per_simd, int iters, float* out, unsigned long long* clk,
        int grid) {
  auto k = rate_kernel<KIND, NACC>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsPad) != hipSuccess)
    return 1;
  const int threads = 4 * 64 * waves_per_simd;
  hipLaunchKernelGGL(k, dim3(grid), dim3(threads), kLdsPad, 0, out, iters / 4, clk, 1);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL(k, dim3(grid), dim3(threads), kLdsPad, 0, out, iters, clk, 2);
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  std::vector<unsigned long long> h(2 * grid);
  if (hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return 1;
  double c = 0.0, r = 0.0;
  for (int b = 0; b < grid; ++b) {
    c += static_cast<double>(h[2 * b]);
    r += static_cast<double>(h[2 * b + 1]);
  }
  c /= grid;
  r /= grid;
  const double mfmas_per_simd = static_cast<double>(waves_per_simd) * iters * NACC;
  const double clk_per_mfma = c / mfmas_per_simd;
  const double flop_clk_cu = 4.0 * flop_of(KIND) / clk_per_mfma;
  const double mhz = r > 0 ? 100.0 * c / r : 0.0;
  const double flop = flop_of(KIND) * mfmas_per_simd * 4.0 * grid;
  const double tflops = flop / (ms * 1e-3) / 1e12;
  const double peak_clk = KIND == kBF16 ? 4096.0 : (KIND == kF32 ? 256.0 : 8192.0);
  printf("case %-22s waves_per_simd %d chains %d clk_per_mfma %.2f flop_per_clk_cu %.0f "
         "mhz %.0f tflops %.1f pct_of_2400mhz_peak %.1f\n",
         name, waves_per_simd, NACC, clk_per_mfma, flop_clk_cu, mhz, tflops,
         100.0 * tflops / (peak_clk * grid * 2.4e9 / 1e12));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

}  // namespace

int main() {
  int grid = 0;
  if (hipDeviceGetAttribute(&grid, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess ||
      grid <= 0)
    return 2;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  if (hipMalloc(&out, static_cast<size_t>(grid) * 512 * sizeof(float)) != hipSuccess ||
      hipMalloc(&clk, static_cast<size_t>(grid) * 2 * sizeof(unsigned long long)) != hipSuccess)
    return 2;
  int rc = 0;
  // throughput: two waves per SIMD, four independent accumulators each
  rc |= run<kBF16, 4>("bf16_16x16x32", 2, 20000, out, clk, grid);
  rc |= run<kFP8, 4>("fp8_16x16x128", 2, 10000, out, clk, grid);
  rc |= run<kFP4xFP8, 4>("fp4xfp8_16x16x128", 2, 10000, out, clk, grid);
  rc |= run<kFP4, 4>("fp4xfp4_16x16x128", 2, 10000, out, clk, grid);
  rc |= run<kF32, 4>("f32_16x16x4", 2, 10000, out, clk, grid);
  // dependent chains: one wave per SIMD, one accumulator
  rc |= run<kBF16, 1>("bf16_chain", 1, 20000, out, clk, grid);
  rc |= run<kF32, 1>("f32_chain", 1, 20000, out, clk, grid);
  rc |= run<kF32, 2>("f32_two_chains", 1, 20000, out, clk, grid);
  const hipError_t e = hipDeviceSynchronize();
  printf("status %d\n", static_cast<int>(e));
  (void)hipFree(out);
  (void)hipFree(clk);
  return (rc || e != hipSuccess) ? 1 : 0;
}
