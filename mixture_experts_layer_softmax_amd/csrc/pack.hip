// pack.hip -- one-time weight re-layout: every expert matrix [K][N] becomes
// its transpose [N][K], so the contraction axis is contiguous and the grouped
// GEMMs read whole 128-byte K rows per weight column.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// 64 x 64 element tile through LDS; blockIdx.z = expert.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src,
                                                        T* __restrict__ dst, int64_t K,
                                                        int64_t N) {
  __shared__ T tile[64][65];
  const int64_t e = blockIdx.z;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * 64, n0 = static_cast<int64_t>(blockIdx.x) * 64;
  const T* s = src + e * K * N;
  T* d = dst + e * K * N;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    if (k0 + r < K && n0 + c < N) tile[r][c] = s[(k0 + r) * N + n0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;  // r: n, c: k
    if (n0 + r < N && k0 + c < K) d[(n0 + r) * K + k0 + c] = tile[c][r];
  }
}

}  // namespace

void launch_pack(int E, int64_t K, int64_t N, int elem_bytes, const void* src, void* dst,
                 hipStream_t s) {
  if (E <= 0 || K <= 0 || N <= 0) return;
  dim3 grid(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((K + 63) / 64),
            static_cast<unsigned>(E));
  if (elem_bytes == 4)
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>(static_cast<const uint32_t*>(src),
                                                    static_cast<uint32_t*>(dst), K, N);
  else if (elem_bytes == 2)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src),
                                                    static_cast<uint16_t*>(dst), K, N);
  else
    transpose_kernel<uint8_t><<<grid, 256, 0, s>>>(static_cast<const uint8_t*>(src),
                                                   static_cast<uint8_t*>(dst), K, N);
}

}  // namespace moe
