// Converts a file of fp32 values to FP8 E4M3 codes with gfx950's
// v_cvt_pk_fp8_f32, after clamping each value to [-448, 448], and writes the
// codes to a second file.  Usage: fp8_convert <in.f32> <out.u8>.  The test
// compares the codes with the oracle's E4M3FN encoder (round to nearest even,
// saturating at 448).  The kernel touches in[0..n) and out[0..n) only
// (n rounded up to pairs on the host, the tail padded with zeros).
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>

__global__ void cvt(const float* __restrict__ in, unsigned short* __restrict__ out, long pairs) {
  for (long i = blockIdx.x * 256l + threadIdx.x; i < pairs; i += 256l * gridDim.x) {
    const float a = fminf(fmaxf(in[2 * i], -448.0f), 448.0f);
    const float b = fminf(fmaxf(in[2 * i + 1], -448.0f), 448.0f);
    out[i] = static_cast<unsigned short>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffff);
  }
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: fp8_convert in.f32 out.u8\n");
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 3;
  fseek(f, 0, SEEK_END);
  const long n = ftell(f) / 4;
  fseek(f, 0, SEEK_SET);
  const long pairs = (n + 1) / 2;
  std::vector<float> h(2 * pairs, 0.0f);
  if (fread(h.data(), 4, n, f) != static_cast<size_t>(n)) return 4;
  fclose(f);
  float* din = nullptr;
  unsigned short* dout = nullptr;
  if (hipMalloc(&din, 8 * pairs) != hipSuccess || hipMalloc(&dout, 2 * pairs) != hipSuccess) return 5;
  if (hipMemcpy(din, h.data(), 8 * pairs, hipMemcpyHostToDevice) != hipSuccess) return 5;
  cvt<<<1024, 256>>>(din, dout, pairs);
  std::vector<unsigned char> q(2 * pairs);
  if (hipMemcpy(q.data(), dout, 2 * pairs, hipMemcpyDeviceToHost) != hipSuccess) return 6;
  FILE* g = fopen(argv[2], "wb");
  if (!g) return 7;
  fwrite(q.data(), 1, n, g);
  fclose(g);
  (void)hipFree(din);
  (void)hipFree(dout);
  return 0;
}
