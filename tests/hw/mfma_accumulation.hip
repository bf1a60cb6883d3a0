// Accumulation precision of the gfx950 MFMAs the expert GEMMs use, measured
// with exact operands: one output element receives one product of 1.0 and
// K-1 products of p = 2^-j (all other elements K products of p, or a mix).
// For each MFMA and j the program prints the fraction of the K-1 small
// products that survive next to the 1.0:  "<mfma> <K> <j> <fraction>".
// Test infrastructure: it characterises the hardware behind the tolerance of
// the FP8 hidden-row check; the library does not use it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// one wave; lane l holds 32 E4M3 bytes of A and of B (K = 128)
__global__ void mfma_f8f6f4(const uint8_t* A, const uint8_t* B, float* C) {
  const int l = threadIdx.x;
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = reinterpret_cast<const int*>(A + 32 * l)[i];
    b[i] = reinterpret_cast<const int*>(B + 32 * l)[i];
  }
  const f32x4 c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
  for (int r = 0; r < 4; ++r) C[4 * l + r] = c[r];
}

// one wave; lane l holds 8 bf16 of A and of B (K = 32)
__global__ void mfma_bf16(const uint16_t* A, const uint16_t* B, float* C) {
  const int l = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(__bf16, A[8 * l + i]);
    b[i] = __builtin_bit_cast(__bf16, B[8 * l + i]);
  }
  const f32x4 c =
      __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  for (int r = 0; r < 4; ++r) C[4 * l + r] = c[r];
}

// E4M3FN code of 2^e, e in [-9, 8]; bf16 bits of 2^e
static uint8_t e4m3_pow2(int e) { return e >= -6 ? uint8_t((e + 7) << 3) : uint8_t(1 << (e + 9)); }
static uint16_t bf16_pow2(int e) { return uint16_t((e + 127) << 7); }

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t r_ = (x);                                                          \
    if (r_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(r_), __LINE__); \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main() {
  uint8_t *dA, *dB;
  float* dC;
  CHECK(hipMalloc(&dA, 2048));
  CHECK(hipMalloc(&dB, 2048));
  CHECK(hipMalloc(&dC, 256 * sizeof(float)));
  std::vector<float> c(256);
  for (int kind = 0; kind < 2; ++kind) {
    const int K = kind == 0 ? 128 : 32;
    const int jmax = kind == 0 ? 18 : 30;  // E4M3 products reach 2^-18
    for (int j = 4; j <= jmax; ++j) {
      const int ja = j / 2, jb = j - ja;    // p = 2^-ja * 2^-jb
      if (kind == 0) {
        std::vector<uint8_t> a(2048, e4m3_pow2(-ja)), b(2048, e4m3_pow2(-jb));
        a[0] = b[0] = e4m3_pow2(0);         // lane 0's first value: row 0, col 0, same k
        CHECK(hipMemcpy(dA, a.data(), 2048, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dB, b.data(), 2048, hipMemcpyHostToDevice));
        mfma_f8f6f4<<<1, 64>>>(dA, dB, dC);
      } else {
        std::vector<uint16_t> a(512, bf16_pow2(-ja)), b(512, bf16_pow2(-jb));
        a[0] = b[0] = bf16_pow2(0);
        CHECK(hipMemcpy(dA, a.data(), 1024, hipMemcpyHostToDevice));
        CHECK(hipMemcpy(dB, b.data(), 1024, hipMemcpyHostToDevice));
        mfma_bf16<<<1, 64>>>(reinterpret_cast<uint16_t*>(dA), reinterpret_cast<uint16_t*>(dB), dC);
      }
      CHECK(hipGetLastError());
      CHECK(hipMemcpy(c.data(), dC, 256 * sizeof(float), hipMemcpyDeviceToHost));
      float big = 0.f;
      for (float v : c) big = std::fmax(big, v);  // element (0, 0): 1 + (K-1) p
      const double p = std::ldexp(1.0, -j);
      std::printf("%s %d %d %.6f\n", kind == 0 ? "f8f6f4" : "bf16", K, j,
                  (static_cast<double>(big) - 1.0) / ((K - 1) * p));
    }
  }
  return 0;
}
