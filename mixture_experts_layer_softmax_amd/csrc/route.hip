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
// x[t][i] and gate_w[i][e] of one hidden chunk already widened to fp32, both
// with the hidden index contiguous, so a lane reads four consecutive i of one
// row with one float4 load and then runs its RT x RE chains four FMA steps, i
// ascending -- the fixed summation order is untouched by the blocking.  The
// next chunk is loaded into registers while the current one is computed.
template <int RT, int RE, int TYL, int TXL, int KB, bool BF16>
__global__ __launch_bounds__(256) void logits_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv,
    const float* __restrict__ bias, float* __restrict__ logits, int T, int d,
    int E) {
  static_assert(TYL * TXL == 256, "256 threads");
  // fma-step unroll of whole chunks for lanes with one chain (its LDS
  // latency is otherwise exposed); blocked shapes keep the plain loop
  constexpr int UNR = (RT * RE == 1) ? 8 : 1;
  constexpr int TT = TYL * RT, TE = TXL * RE;
  constexpr int LD = KB + kRoutePad;
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte global load
  constexpr int XCH = TT * (KB / EPC), WCH = KB * (TE / EPC);  // 16-byte chunks
  constexpr int XR = (XCH + 255) / 256, WR = (WCH + 255) / 256;
  extern __shared__ __attribute__((aligned(16))) float route_lds[];
  float (*xs)[LD] = reinterpret_cast<float (*)[LD]>(route_lds);            // [TT][LD]
  float (*ws)[LD] = reinterpret_cast<float (*)[LD]>(route_lds + TT * LD);  // [TE][LD]
  const int tid = threadIdx.x, tx = tid % TXL, ty = tid / TXL;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  float acc[RT][RE];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b) acc[a][b] = 0.0f;

  // prefetch registers: raw 16-byte pieces of the next chunk (widened when
  // stored to LDS); out-of-range pieces are zero
  u32x4 xr[XR], wr[WR];
  bool wvec[WR];  // piece loaded as one aligned 16-byte vector
#define MOE_RLOAD(I0)                                                                    \
  do {                                                                                   \
    _Pragma("unroll") for (int r = 0; r < XR; ++r) {                                     \
      const int idx = tid + 256 * r;                                                     \
      const int tl = idx / (KB / EPC), il = (idx % (KB / EPC)) * EPC;                    \
      const int t = t0 + tl, i = (I0) + il;                                              \
      xr[r] = u32x4{0u, 0u, 0u, 0u};                                                     \
      if (idx < XCH && t < T && i < d) {                                                 \
        const size_t o = static_cast<size_t>(t) * d + i;                                 \
        xr[r] = BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(xv) + o) \
                     : *reinterpret_cast<const u32x4*>(static_cast<const float*>(xv) + o); \
      }                                                                                  \
    }                                                                                    \
    _Pragma("unroll") for (int r = 0; r < WR; ++r) {                                     \
      const int idx = tid + 256 * r;                                                     \
      const int il = idx / (TE / EPC), el = (idx % (TE / EPC)) * EPC;                    \
      const int e = e0 + el, i = (I0) + il;                                              \
      wr[r] = u32x4{0u, 0u, 0u, 0u};                                                     \
      wvec[r] = idx < WCH && i < d && E % EPC == 0 && e + EPC <= E;                      \
      if (wvec[r]) {                                                                     \
        const size_t o = static_cast<size_t>(i) * E + e;                                 \
        wr[r] = BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(wv) + o) \
                     : *reinterpret_cast<const u32x4*>(static_cast<const float*>(wv) + o); \
      }                                                                                  \
    }                                                                                    \
  } while (0)
#define MOE_RSTORE(I0)                                                                   \
  do {                                                                                   \
    _Pragma("unroll") for (int r = 0; r < XR; ++r) {                                     \
      const int idx = tid + 256 * r;                                                     \
      if (idx < XCH) {                                                                   \
        const int tl = idx / (KB / EPC), il = (idx % (KB / EPC)) * EPC;                  \
        float v[EPC];                                                                    \
        if (BF16) {                                                                      \
          _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                \
            v[2 * q] = __uint_as_float(xr[r][q] << 16);                                  \
            v[2 * q + 1] = __uint_as_float(xr[r][q] & 0xffff0000u);                      \
          }                                                                              \
        } else {                                                                         \
          _Pragma("unroll") for (int q = 0; q < EPC; ++q) v[q] = __uint_as_float(xr[r][q]); \
        }                                                                                \
        _Pragma("unroll") for (int q = 0; q < EPC; q += 4) *reinterpret_cast<f32x4*>(    \
            &xs[tl][il + q]) = f32x4{v[q], v[q + 1], v[q + 2], v[q + 3]};                \
      }                                                                                  \
    }                                                                                    \
    _Pragma("unroll") for (int r = 0; r < WR; ++r) {                                     \
      const int idx = tid + 256 * r;                                                     \
      if (idx < WCH) {                                                                   \
        const int il = idx / (TE / EPC), el = (idx % (TE / EPC)) * EPC;                  \
        const int i = (I0) + il;                                                         \
        float v[EPC];                                                                    \
        if (wvec[r]) {                                                                   \
          if (BF16) {                                                                    \
            _Pragma("unroll") for (int q = 0; q < 4; ++q) {                              \
              v[2 * q] = __uint_as_float(wr[r][q] << 16);                                \
              v[2 * q + 1] = __uint_as_float(wr[r][q] & 0xffff0000u);                    \
            }                                                                            \
          } else {                                                                       \
            _Pragma("unroll") for (int q = 0; q < EPC; ++q) v[q] = __uint_as_float(wr[r][q]); \
          }                                                                              \
        } else {                                                                         \
          _Pragma("unroll") for (int q = 0; q < EPC; ++q) {                              \
            const int eq = e0 + el + q;                                                  \
            float val = 0.0f;                                                            \
            if (i < d && eq < E) {                                                       \
              const size_t o = static_cast<size_t>(i) * E + eq;                          \
              val = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(wv)[o])              \
                         : static_cast<const float*>(wv)[o];                             \
            }                                                                            \
            v[q] = val;                                                                  \
          }                                                                              \
        }                                                                                \
        _Pragma("unroll") for (int q = 0; q < EPC; ++q) ws[el + q][il] = v[q];           \
      }                                                                                  \
    }                                                                                    \
  } while (0)

  MOE_RLOAD(0);
  for (int i0 = 0; i0 < d; i0 += KB) {
    MOE_RSTORE(i0);
    __syncthreads();
    if (i0 + KB < d) MOE_RLOAD(i0 + KB);  // in flight during this chunk's FMAs
    const int iend = min(KB, d - i0);     // d % 8 == 0, so iend % 4 == 0
#define MOE_GATE_STEP(IL)                                                                 \
  do {                                                                                    \
    f32x4 xv4[RT], wv4[RE];                                                               \
    _Pragma("unroll") for (int a = 0; a < RT; ++a) xv4[a] =                               \
        *reinterpret_cast<const f32x4*>(&xs[ty * RT + a][(IL)]);                          \
    _Pragma("unroll") for (int b = 0; b < RE; ++b) wv4[b] =                               \
        *reinterpret_cast<const f32x4*>(&ws[tx * RE + b][(IL)]);                          \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                         \
    _Pragma("unroll") for (int a = 0; a < RT; ++a)                                        \
    _Pragma("unroll") for (int b = 0; b < RE; ++b) acc[a][b] =                            \
        __builtin_fmaf(xv4[a][u], wv4[b][u], acc[a][b]);                                  \
  } while (0)
    if (UNR > 1 && iend == KB) {
      // whole chunk: a compile-time trip count, unrolled so that the LDS
      // reads of the next steps are issued ahead of this step's fma chain
      // (the fma order of every chain stays i ascending)
#pragma unroll UNR
      for (int il = 0; il < KB; il += 4) MOE_GATE_STEP(il);
    } else {
      for (int il = 0; il < iend; il += 4) MOE_GATE_STEP(il);
    }
#undef MOE_GATE_STEP
    __syncthreads();
  }
#undef MOE_RLOAD
#undef MOE_RSTORE
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
  // Largest register blocking that still gives the chip >= 1024 workgroups
  // (four per CU: the chains are latency-bound, measured) and does not leave
  // most expert lanes idle.
  struct Cfg {
    int rt, re, tyl, txl;
  };
  // KB (hidden chunk per LDS tile) is 64 for the most blocked shapes (more
  // FMAs per chunk) and 128 otherwise, so a chunk's FMAs cover the global
  // load latency of the next one.
  static constexpr Cfg cfgs[] = {{8, 4, 16, 16}, {4, 4, 16, 16}, {2, 4, 32, 8},
                                 {2, 2, 16, 16}, {1, 2, 32, 8},  {1, 1, 16, 16}};
  int pick = 5;
  for (int c = 0; c < 5; ++c) {
    const int TT = cfgs[c].tyl * cfgs[c].rt, TE = cfgs[c].txl * cfgs[c].re;
    const long long wgs = static_cast<long long>((T + TT - 1) / TT) * ((E + TE - 1) / TE);
    if (TE <= E && wgs >= 1024) {  // four or more workgroups per CU
      pick = c;
      break;
    }
  }
  auto go = [&](auto kern, int TT, int TE, int KB) {
    dim3 grid((T + TT - 1) / TT, (E + TE - 1) / TE);
    const size_t lds = sizeof(float) * static_cast<size_t>(TT + TE) * (KB + kRoutePad);
    kern<<<grid, 256, lds, s>>>(x, gate_w, bias, logits, T, d, E);
  };
#define MOE_L(C, RT, RE, TYL, TXL, KB)                                                    \
  if (pick == C) {                                                                        \
    if (bf16)                                                                             \
      go(logits_kernel<RT, RE, TYL, TXL, KB, true>, TYL * RT, TXL * RE, KB);              \
    else                                                                                  \
      go(logits_kernel<RT, RE, TYL, TXL, KB, false>, TYL * RT, TXL * RE, KB);             \
    return;                                                                               \
  }
  MOE_L(0, 8, 4, 16, 16, 64)
  MOE_L(1, 4, 4, 16, 16, 64)
  MOE_L(2, 2, 4, 32, 8, 128)
  MOE_L(3, 2, 2, 16, 16, 128)
  MOE_L(4, 1, 2, 32, 8, 128)
  MOE_L(5, 1, 1, 16, 16, 128)
#undef MOE_L
}

void launch_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                 hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, T, E, k);
}

}  // namespace moe
