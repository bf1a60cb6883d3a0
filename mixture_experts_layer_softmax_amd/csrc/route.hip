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

constexpr int kRoutePad = 4;  // floats of padding per LDS row (keeps float4 alignment)

// Block of 256 threads = TYL x TXL lanes; lane (ty, tx) owns tokens
// t0 + ty * RT + a (a < RT) and experts e0 + tx * RE + b (b < RE).  LDS holds
// x[t][i] and gate_w[i][e] of the chunk already widened to fp32, both with the
// hidden index contiguous, so a lane reads four consecutive i of one row with
// one float4 load and then runs its RT x RE chains four FMA steps, i
// ascending -- the fixed summation order is untouched by the blocking.
template <int RT, int RE, int TYL, int TXL, int kRouteKB, bool BF16>
__global__ __launch_bounds__(256) void logits_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv,
    const float* __restrict__ bias, float* __restrict__ logits, int T, int d,
    int E) {
  static_assert(TYL * TXL == 256, "256 threads");
  constexpr int TT = TYL * RT, TE = TXL * RE;
  constexpr int LD = kRouteKB + kRoutePad;
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte global load
  __shared__ __attribute__((aligned(16))) float xs[TT][LD];  // [token][i]
  __shared__ __attribute__((aligned(16))) float ws[TE][LD];  // [expert][i]
  const int tid = threadIdx.x, tx = tid % TXL, ty = tid / TXL;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  float acc[RT][RE];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b) acc[a][b] = 0.0f;

  for (int i0 = 0; i0 < d; i0 += kRouteKB) {
    // x chunk: TT rows of KB elements, 16-byte loads along i
    for (int idx = tid; idx < TT * (kRouteKB / EPC); idx += 256) {
      const int tl = idx / (kRouteKB / EPC), il = (idx % (kRouteKB / EPC)) * EPC;
      const int t = t0 + tl, i = i0 + il;
      float v[EPC];
      if (t < T && i < d) {
        const size_t o = static_cast<size_t>(t) * d + i;
        if (BF16) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(xv) + o);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(raw[q] << 16);
            v[2 * q + 1] = __uint_as_float(raw[q] & 0xffff0000u);
          }
        } else {
          const f32x4 raw = *reinterpret_cast<const f32x4*>(static_cast<const float*>(xv) + o);
#pragma unroll
          for (int q = 0; q < EPC; ++q) v[q] = raw[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < EPC; ++q) v[q] = 0.0f;
      }
#pragma unroll
      for (int q = 0; q < EPC; q += 4)
        *reinterpret_cast<f32x4*>(&xs[tl][il + q]) = f32x4{v[q], v[q + 1], v[q + 2], v[q + 3]};
    }
    // gate_w chunk: KB rows of TE experts (expert index contiguous in
    // memory), stored transposed so the hidden index is contiguous in LDS
    for (int idx = tid; idx < kRouteKB * (TE / EPC); idx += 256) {
      const int il = idx / (TE / EPC), el = (idx % (TE / EPC)) * EPC;
      const int e = e0 + el, i = i0 + il;
      float v[EPC];
      if (i < d && E % EPC == 0 && e + EPC <= E) {  // aligned 16-byte load
        const size_t o = static_cast<size_t>(i) * E + e;
        if (BF16) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(wv) + o);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(raw[q] << 16);
            v[2 * q + 1] = __uint_as_float(raw[q] & 0xffff0000u);
          }
        } else {
          const f32x4 raw = *reinterpret_cast<const f32x4*>(static_cast<const float*>(wv) + o);
#pragma unroll
          for (int q = 0; q < EPC; ++q) v[q] = raw[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int eq = e + q;
          float val = 0.0f;
          if (i < d && eq < E) {
            const size_t o = static_cast<size_t>(i) * E + eq;
            val = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(wv)[o])
                       : static_cast<const float*>(wv)[o];
          }
          v[q] = val;
        }
      }
#pragma unroll
      for (int q = 0; q < EPC; ++q) ws[el + q][il] = v[q];
    }
    __syncthreads();
    const int iend = min(kRouteKB, d - i0);  // d % 8 == 0, so iend % 4 == 0
    for (int il = 0; il < iend; il += 4) {
      f32x4 xr[RT], wr[RE];
#pragma unroll
      for (int a = 0; a < RT; ++a) xr[a] = *reinterpret_cast<const f32x4*>(&xs[ty * RT + a][il]);
#pragma unroll
      for (int b = 0; b < RE; ++b) wr[b] = *reinterpret_cast<const f32x4*>(&ws[tx * RE + b][il]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
          for (int b = 0; b < RE; ++b) acc[a][b] = __builtin_fmaf(xr[a][u], wr[b][u], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < RT; ++a) {
    const int t = t0 + ty * RT + a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < RE; ++b) {
      const int e = e0 + tx * RE + b;
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
  // Largest register blocking that still gives the chip >= 256 workgroups
  // and does not leave most expert lanes idle.
  struct Cfg {
    int rt, re, tyl, txl;
  };
  // KB (hidden chunk per LDS tile) is 32 for the blocked shapes and 128 for
  // the one-output-per-lane shapes of small T, where per-chunk latency
  // dominates.
  static constexpr Cfg cfgs[] = {{8, 4, 16, 16}, {4, 4, 16, 16}, {2, 4, 32, 8},
                                 {2, 2, 16, 16}, {1, 2, 32, 8},  {1, 1, 16, 16}};
  int pick = 5;
  for (int c = 0; c < 5; ++c) {
    const int TT = cfgs[c].tyl * cfgs[c].rt, TE = cfgs[c].txl * cfgs[c].re;
    const long long wgs = static_cast<long long>((T + TT - 1) / TT) * ((E + TE - 1) / TE);
    if (TE <= E && wgs >= 512) {  // two or more workgroups per CU
      pick = c;
      break;
    }
  }
  auto go = [&](auto kern, int TT, int TE) {
    dim3 grid((T + TT - 1) / TT, (E + TE - 1) / TE);
    kern<<<grid, 256, 0, s>>>(x, gate_w, bias, logits, T, d, E);
  };
#define MOE_L(C, RT, RE, TYL, TXL, KB)                                                    \
  if (pick == C) {                                                                        \
    if (bf16)                                                                             \
      go(logits_kernel<RT, RE, TYL, TXL, KB, true>, TYL * RT, TXL * RE);                  \
    else                                                                                  \
      go(logits_kernel<RT, RE, TYL, TXL, KB, false>, TYL * RT, TXL * RE);                 \
    return;                                                                               \
  }
  MOE_L(0, 8, 4, 16, 16, 32)
  MOE_L(1, 4, 4, 16, 16, 32)
  MOE_L(2, 2, 4, 32, 8, 32)
  MOE_L(3, 2, 2, 16, 16, 32)
  MOE_L(4, 1, 2, 32, 8, 128)
  MOE_L(5, 1, 1, 16, 16, 128)
#undef MOE_L
}

void launch_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                 hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, T, E, k);
}

}  // namespace moe
