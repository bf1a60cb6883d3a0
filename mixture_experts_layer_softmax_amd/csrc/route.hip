// route.hip -- the gate: router logits, top-k selection and renormalised
// softmax weights (first stage of the layer named on the FlashMoE Kernel
// page, opening paragraph; the gate math itself is the stated workload's
// "renormalised top-k softmax").
//
// Logits follow one fixed fp32 order so the selection is reproducible bit for
// bit on any device: acc = +0, acc = fma(x[t][i], w[i][e], acc) for i
// ascending, then acc + bias[e].  Each logit is one lane's sequential chain;
// parallelism comes from the T x E outputs, register-blocked RT x RE per lane
// over LDS tiles that hold x and gate_w already widened to fp32.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRouteKB = 32;  // hidden-dim chunk staged per LDS tile

// Block of 256 threads = 16 x 16 lanes; lane (ty, tx) owns tokens
// t0 + ty + 16 a (a < RT) and experts e0 + tx + 16 b (b < RE).
template <int RT, int RE, bool BF16>
__global__ __launch_bounds__(256) void logits_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv,
    const float* __restrict__ bias, float* __restrict__ logits, int T, int d,
    int E) {
  constexpr int TT = 16 * RT, TE = 16 * RE;
  __shared__ float xs[kRouteKB][TT + 1];  // [i][token]
  __shared__ float ws[kRouteKB][TE + 1];  // [i][expert]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  float acc[RT][RE];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b) acc[a][b] = 0.0f;

  for (int i0 = 0; i0 < d; i0 += kRouteKB) {
    // stage x[t0 .. t0+TT)[i0 .. i0+KB) transposed, and w[i0 ..][e0 ..)
    for (int idx = tid; idx < TT * kRouteKB; idx += 256) {
      int tl = idx / kRouteKB, il = idx % kRouteKB;
      int t = t0 + tl, i = i0 + il;
      float v = 0.0f;
      if (t < T && i < d) {
        size_t o = static_cast<size_t>(t) * d + i;
        v = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(xv)[o])
                 : static_cast<const float*>(xv)[o];
      }
      xs[il][tl] = v;
    }
    for (int idx = tid; idx < TE * kRouteKB; idx += 256) {
      int il = idx / TE, el = idx % TE;
      int e = e0 + el, i = i0 + il;
      float v = 0.0f;
      if (e < E && i < d) {
        size_t o = static_cast<size_t>(i) * E + e;
        v = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(wv)[o])
                 : static_cast<const float*>(wv)[o];
      }
      ws[il][el] = v;
    }
    __syncthreads();
    const int iend = min(kRouteKB, d - i0);
    for (int il = 0; il < iend; ++il) {
      float xr[RT], wr[RE];
#pragma unroll
      for (int a = 0; a < RT; ++a) xr[a] = xs[il][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < RE; ++b) wr[b] = ws[il][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b = 0; b < RE; ++b) acc[a][b] = __builtin_fmaf(xr[a], wr[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < RT; ++a) {
    int t = t0 + ty + 16 * a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < RE; ++b) {
      int e = e0 + tx + 16 * b;
      if (e >= E) continue;
      float l = acc[a][b];
      if (bias) l = l + bias[e];
      logits[static_cast<size_t>(t) * E + e] = l;
    }
  }
}

// One wavefront per token: k rounds of a wave-wide argmax ordered by
// (logit descending, expert index ascending), then fp64 softmax over the k
// selected logits.  E <= 1024 (16 logits per lane).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int T,
                                                   int E, int k) {
  constexpr int kMaxPerLane = 16;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + static_cast<size_t>(t) * E;
  float v[kMaxPerLane];
#pragma unroll
  for (int s = 0; s < kMaxPerLane; ++s) {
    int e = lane + 64 * s;
    v[s] = (e < E) ? l[e] : -INFINITY;
  }
  int32_t* out_ids = ids + static_cast<size_t>(t) * k;
  float* out_w = w + static_cast<size_t>(t) * k;
  // selection j is kept by lane (j mod 64) in slot j / 64
  int sel_e[kMaxPerLane];
  float sel_v[kMaxPerLane];
  float top0 = 0.0f;
  double sum = 0.0;
  uint32_t taken = 0;  // bit s set: v[s] of this lane already selected
  for (int j = 0; j < k; ++j) {
    // local best among untaken entries (ties: smaller e, i.e. smaller s)
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < kMaxPerLane; ++s) {
      int e = lane + 64 * s;
      bool ok = e < E && !((taken >> s) & 1u);
      if (ok && (be == 0x7fffffff || v[s] > bv || (v[s] == bv && e < be))) {
        bv = v[s];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      bool take = (oe != 0x7fffffff) &&
                  (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (j == 0) top0 = bv;
    sum += exp(static_cast<double>(bv) - static_cast<double>(top0));
#pragma unroll
    for (int s = 0; s < kMaxPerLane; ++s)
      if (j == lane + 64 * s) {
        sel_e[s] = be;
        sel_v[s] = bv;
      }
  }
#pragma unroll
  for (int s = 0; s < kMaxPerLane; ++s) {
    int j = lane + 64 * s;
    if (j < k) {
      double u = exp(static_cast<double>(sel_v[s]) - static_cast<double>(top0));
      out_ids[j] = sel_e[s];
      out_w[j] = static_cast<float>(u / sum);
    }
  }
}

}  // namespace

void launch_logits(const void* x, const void* gate_w, const float* bias, float* logits,
                   int T, int d, int E, bool bf16, hipStream_t s) {
  // Enough blocks to fill the chip first, then the largest register blocking.
  auto go = [&](auto rt, auto re) {
    constexpr int RT = decltype(rt)::value, RE = decltype(re)::value;
    dim3 grid((T + 16 * RT - 1) / (16 * RT), (E + 16 * RE - 1) / (16 * RE));
    if (bf16)
      logits_kernel<RT, RE, true><<<grid, 256, 0, s>>>(x, gate_w, bias, logits, T, d, E);
    else
      logits_kernel<RT, RE, false><<<grid, 256, 0, s>>>(x, gate_w, bias, logits, T, d, E);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  const long long big = static_cast<long long>(T) * E;
  if (big >= (1ll << 22) && E >= 64)
    go(I4{}, I4{});
  else if (big >= (1ll << 20))
    go(I4{}, I2{});
  else if (big >= (1ll << 17))
    go(I2{}, I1{});
  else
    go(I1{}, I1{});
}

void launch_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                 hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, T, E, k);
}

}  // namespace moe
