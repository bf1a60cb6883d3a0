// Main-loop microbenchmark of the grouped GEMM's 256 x 256 bf16 block tile:
// two LDS stages of 64 contraction elements (128-byte rows, the GEMM's XOR
// swizzle), eight waves of 128 x 64, the same fragment reads and 16x16x32
// MFMAs per stage, one barrier per stage.  Global memory is touched only by
// the optional DMA, whose sources stay inside a 4 MB buffer (L2-resident),
// issued in the GEMM's buffer form (buffer_load_dwordx4 ... lds).  Each mode
// drops parts of the loop, to see what bounds it:
//   MODE bit 0: fragment reads from LDS   bit 1: MFMAs   bit 2: stage DMA
// Output, one line per mode: shader clocks per stage (wave 0 of each
// workgroup, s_memtime; the MFMA floor is 2048 at two waves per SIMD), and
// the achieved rate against the 2516.6 TFLOP/s bf16 peak (2.4 GHz).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

namespace {

constexpr int kRowBytes = 128;                  // contraction bytes per row and stage
constexpr int kStage = 2 * 256 * kRowBytes;     // 256 A rows + 256 B rows
constexpr int kWM = 2, kWN = 4, kWaves = kWM * kWN;
constexpr int kTM = 256 / kWM / 16, kTN = 256 / kWN / 16;  // 16 x 16 fragments per wave
constexpr int kSrcBytes = 4 << 20;

__device__ __forceinline__ int swz(int r, int chunk) {
  return r * kRowBytes + ((chunk ^ ((r >> 1) & 7)) << 4);
}

template <int MODE>
__global__ __launch_bounds__(kWaves * 64) void loop_bench(const uint8_t* src, float* out,
                                                          int stages,
                                                          unsigned long long* clk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int l16 = lane & 15, lg = lane >> 4;
  for (int i = tid * 16; i < 2 * kStage; i += kWaves * 64 * 16)
    *reinterpret_cast<uint4*>(lds + i) = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  f32x4 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, kSrcBytes, 0x00020000);
  const uint32_t lane_off = static_cast<uint32_t>(lane * 16 + wave * 4096);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int s = 0; s < stages; ++s) {
    const uint8_t* A = lds + (s & 1) * kStage;
    const uint8_t* B = A + 256 * kRowBytes;
    if constexpr (MODE & 4) {  // the next stage: 64 wave-wide DMAs of 1 KB
      uint8_t* dst = lds + ((s + 1) & 1) * kStage;
#pragma unroll
      for (int q = 0; q < 64 / kWaves; ++q) {
        const uint32_t off = (lane_off + static_cast<uint32_t>(s) * 65536u +
                              static_cast<uint32_t>(q) * 1024u * kWaves) & (kSrcBytes - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(dst + (wave + kWaves * q) * 1024), 16,
            off, 0, 0, 0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {  // two 16x16x32 k-steps per stage
      bf16x8 wf[kTN], xf[kTM];
      if constexpr (MODE & 1) {
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          wf[j] = *reinterpret_cast<const bf16x8*>(B + swz(wn * 64 + 16 * j + l16, kk * 4 + lg));
#pragma unroll
        for (int i = 0; i < kTM; ++i)
          xf[i] = *reinterpret_cast<const bf16x8*>(A + swz(wm * 128 + 16 * i + l16, kk * 4 + lg));
      } else {  // operands from registers
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
          for (int q = 0; q < 8; ++q) wf[j][q] = static_cast<__bf16>(static_cast<float>(lane + j + q + kk));
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int q = 0; q < 8; ++q) xf[i][q] = static_cast<__bf16>(static_cast<float>(lane - i + q));
      }
      if constexpr (MODE & 2) {
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
      } else {  // keep the reads alive
#pragma unroll
        for (int i = 0; i < kTM; ++i) acc[i][0][0] += static_cast<float>(xf[i][0]);
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[0][j][1] += static_cast<float>(wf[j][1]);
      }
      if constexpr ((MODE & 3) == 3) {  // every read of the step before its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, kTM + kTN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, kTM * kTN, 0);
      }
    }
    if constexpr (MODE & 4) __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[blockIdx.x * blockDim.x + tid] = sum;
  if (tid == 0) clk[blockIdx.x] = t1 - t0;
}

template <int MODE>
int run(const char* name, const uint8_t* src, float* out, unsigned long long* clk, int grid) {
  auto k = loop_bench<MODE>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStage) != hipSuccess)
    return 1;
  const int stages = 2000;
  hipLaunchKernelGGL(k, dim3(grid), dim3(kWaves * 64), 2 * kStage, 0, src, out, stages, clk);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL(k, dim3(grid), dim3(kWaves * 64), 2 * kStage, 0, src, out, stages, clk);
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  std::vector<unsigned long long> h(grid);
  if (hipMemcpy(h.data(), clk, grid * sizeof(unsigned long long), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return 1;
  double avg = 0.0;
  for (unsigned long long v : h) avg += static_cast<double>(v);
  avg /= grid;
  const double flop = 2.0 * 256 * 256 * 64 * stages * grid;  // per stage: 256 x 256 x 64
  const double tflops = (MODE & 2) ? flop / (ms * 1e-3) / 1e12 : 0.0;
  printf("mode %d %-24s clk_per_stage %.1f tflops %.0f pct_of_peak %.1f\n", MODE, name,
         avg / stages, tflops, tflops / 25.166);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

}  // namespace

int main() {
  const int grid = 256;  // one workgroup per CU
  uint8_t* src = nullptr;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  if (hipMalloc(&src, kSrcBytes) != hipSuccess || hipMalloc(&out, grid * 512 * sizeof(float)) ||
      hipMalloc(&clk, grid * sizeof(unsigned long long)))
    return 2;
  if (hipMemset(src, 1, kSrcBytes) != hipSuccess) return 2;
  int rc = 0;
  rc |= run<2>("mfma_only", src, out, clk, grid);
  rc |= run<1>("reads_only", src, out, clk, grid);
  rc |= run<3>("reads_mfma", src, out, clk, grid);
  rc |= run<5>("reads_dma", src, out, clk, grid);
  rc |= run<6>("mfma_dma", src, out, clk, grid);
  rc |= run<7>("reads_mfma_dma", src, out, clk, grid);
  const hipError_t e = hipDeviceSynchronize();
  printf("status %d\n", static_cast<int>(e));
  (void)hipFree(src);
  (void)hipFree(out);
  (void)hipFree(clk);
  return (rc || e != hipSuccess) ? 1 : 0;
}
