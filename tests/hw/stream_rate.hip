// Streaming rates of the memory paths the layer's kernels use, measured
// with nothing else running:
//   hbm_read_gW_uU  every lane streams 16-byte loads over a 2 GiB buffer
//                 (far larger than L2 + the 256 MB MALL), grid-stride, each
//                 element read once per pass, W workgroups of 4 waves per
//                 CU and U loads in flight per lane ("nt": non-temporal
//                 hint): the read rate HBM delivers to plain vector loads.
//   hbm_dma_lds   the same bytes through direct global->LDS loads in the
//                 buffer form the GEMMs use (buffer_load_dwordx4 ... lds),
//                 a 16 KB LDS window per workgroup, eight loads in flight
//                 per wave before each wait.
//   lds_read      ds_read_b128 of a 64 KB LDS buffer by 16 waves per CU,
//                 conflict-free addresses (lane L reads the 16 bytes at
//                 16 L of a 1 KB block), no global memory: bytes per shader
//                 clock per CU.
// Output, one line per case: "case NAME bytes B ms T tbps R" (lds_read:
// "case lds_read bytes_per_clk_cu X mhz M").
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

namespace {

constexpr size_t kBytes = size_t{2} << 30;  // 2 GiB
constexpr size_t kElems = kBytes / 16;
constexpr int kThreads = 256;
constexpr int kDmaWindow = 16 * 1024;

template <int UNROLL, bool NT>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                        unsigned* __restrict__ out) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  // UNROLL independent loads in flight per lane
  for (; i + (UNROLL - 1) * stride < kElems; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < kElems; i += stride) acc ^= src[i];
  out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kThreads) void dma_kernel(const uint8_t* __restrict__ src,
                                                       unsigned* __restrict__ out,
                                                       uint32_t rounds) {
  extern __shared__ __attribute__((aligned(16))) uint8_t win[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, 0x7fffffff, 0x00020000);
  // a workgroup moves 16 KB per round (4 waves x 4 loads of 1 KB); rounds
  // (a multiple of twice the grid, all below the buffer resource's 2^31 - 1
  // byte reach) are grid-strided, two rounds in flight before each wait
  constexpr uint32_t kRound = kDmaWindow;
  const uint32_t stride = gridDim.x;
  unsigned acc = 0;
  uint32_t r = blockIdx.x;
  for (; r + stride < rounds; r += 2 * stride) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t base = (r + h * stride) * kRound;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int blk = wave * 2 + q;  // 1 KB block of the half window
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(win + h * (kRound / 2) + blk * 1024),
            16, base + static_cast<uint32_t>(blk * 2 * 1024 + lane * 16), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc,
            (__attribute__((address_space(3))) void*)(win + h * (kRound / 2) + blk * 1024),
            16, base + static_cast<uint32_t>(blk * 2 * 1024 + 1024 + lane * 16), 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
    acc ^= reinterpret_cast<const unsigned*>(win)[tid];
    __syncthreads();
  }
  out[static_cast<size_t>(blockIdx.x) * kThreads + tid] = acc;
}

constexpr int kLdsThreads = 1024;  // 16 waves, one workgroup per CU

__global__ __launch_bounds__(kLdsThreads) void lds_kernel(unsigned* __restrict__ out, int iters,
                                                          unsigned long long* clk) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[64 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < 64 * 1024; i += kLdsThreads * 16)
    *reinterpret_cast<u32x4*>(buf + i) = u32x4{static_cast<unsigned>(i), 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    // 16 reads per wave per iteration, 1 KB each, the block moving with the
    // iteration (so that no read is loop-invariant); the xor chain keeps
    // every read alive
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc ^= *reinterpret_cast<const u32x4*>(buf + ((wave * 16 + j + it) & 63) * 1024 +
                                             lane * 16);
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  out[static_cast<size_t>(blockIdx.x) * kLdsThreads + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

int time_launch(const char* name, void (*launch)(void*, unsigned*, int), void* src,
                unsigned* out, int grid, double bytes) {
  launch(src, out, grid);  // warm-up
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  const int reps = 5;
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r) launch(src, out, grid);
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  ms /= reps;
  printf("case %-12s bytes %.0f ms %.4f tbps %.3f\n", name, bytes, ms, bytes / (ms * 1e-3) / 1e12);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

template <int UNROLL, bool NT>
void launch_read(void* src, unsigned* out, int grid) {
  hipLaunchKernelGGL((read_kernel<UNROLL, NT>), dim3(grid), dim3(kThreads), 0, 0,
                     static_cast<const u32x4*>(src), out);
}
uint32_t dma_rounds(int grid) {
  const uint32_t reach = (0x7fffffffu - kDmaWindow) / kDmaWindow;
  return reach / (2u * grid) * (2u * grid);
}
void launch_dma(void* src, unsigned* out, int grid) {
  hipLaunchKernelGGL(dma_kernel, dim3(grid), dim3(kThreads), kDmaWindow, 0,
                     static_cast<const uint8_t*>(src), out, dma_rounds(grid));
}

}  // namespace

int main() {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess ||
      cus <= 0)
    return 2;
  const int grid = cus * 8;
  const int max_grid = cus * 32;
  void* src = nullptr;
  unsigned* out = nullptr;
  unsigned long long* clk = nullptr;
  if (hipMalloc(&src, kBytes) != hipSuccess ||
      hipMalloc(&out, static_cast<size_t>(max_grid) * kThreads * sizeof(unsigned)) != hipSuccess ||
      hipMalloc(&clk, static_cast<size_t>(grid) * 2 * sizeof(unsigned long long)) != hipSuccess)
    return 2;
  if (hipMemset(src, 0x5a, kBytes) != hipSuccess) return 2;
  int rc = 0;
  // plain loads: workgroups per CU x loads in flight per lane, with and
  // without the non-temporal hint
  char name[64];
  for (int wpc : {4, 8, 16, 32}) {
    snprintf(name, sizeof(name), "hbm_read_g%d_u4", wpc);
    rc |= time_launch(name, launch_read<4, false>, src, out, cus * wpc, static_cast<double>(kBytes));
    snprintf(name, sizeof(name), "hbm_read_g%d_u8", wpc);
    rc |= time_launch(name, launch_read<8, false>, src, out, cus * wpc, static_cast<double>(kBytes));
    snprintf(name, sizeof(name), "hbm_read_g%d_u4nt", wpc);
    rc |= time_launch(name, launch_read<4, true>, src, out, cus * wpc, static_cast<double>(kBytes));
  }
  const double dma_bytes = static_cast<double>(dma_rounds(grid)) * kDmaWindow;
  rc |= time_launch("hbm_dma_lds", launch_dma, src, out, grid, dma_bytes);
  // LDS: one workgroup of 16 waves per CU (its 64 KB buffer and 1024
  // threads), every wave reading 16 KB per iteration
  const int iters = 4000;
  hipLaunchKernelGGL(lds_kernel, dim3(cus), dim3(kLdsThreads), 0, 0, out, iters, clk);
  if (hipDeviceSynchronize() != hipSuccess) return 1;
  std::vector<unsigned long long> h(2 * static_cast<size_t>(cus));
  if (hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return 1;
  double c = 0.0, r = 0.0;
  for (int b = 0; b < cus; ++b) {
    c += static_cast<double>(h[2 * b]);
    r += static_cast<double>(h[2 * b + 1]);
  }
  c /= cus;
  r /= cus;
  const double per_cu_bytes = 16.0 * 16 * 1024 * static_cast<double>(iters);
  printf("case %-12s bytes_per_clk_cu %.1f mhz %.0f\n", "lds_read", per_cu_bytes / c,
         r > 0 ? 100.0 * c / r : 0.0);
  const hipError_t e = hipDeviceSynchronize();
  printf("status %d\n", static_cast<int>(e));
  (void)hipFree(src);
  (void)hipFree(out);
  (void)hipFree(clk);
  return (rc || e != hipSuccess) ? 1 : 0;
}
