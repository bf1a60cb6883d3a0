// route.hip -- the gate: router logits, top-k selection and renormalised
// softmax weights (first stage of the layer named on the FlashMoE Kernel
// page, opening paragraph; the gate math itself is the stated workload's
// "renormalised top-k softmax").
//
// Logits follow one fixed fp32 order so the selection is reproducible bit for
// bit on any device: acc = +0, acc = fma(x[t][i], w[i][e], acc) for i
// ascending, then acc + bias[e].  The chains run on the fp32 MFMA, whose
// four-product step is exactly four such fmas in order (see gate_kernel).
#include "device_common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace moe {

namespace {

// Top-k of one token's E logits l[0..E) (global or LDS) by one wavefront: k
// rounds of a wave-wide argmax ordered by (logit descending, expert index
// ascending), then the softmax over the k selected logits in fp64 (lane j
// evaluates exp(l_j - l_0) of selection j; the sum is a wave reduction).
// E <= 64 * SLOTS.
template <int SLOTS>
__device__ __forceinline__ void topk_row(const float* l, int E, int k, int32_t* out_ids,
                                         float* out_w, int lane) {
  float v[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    int e = lane + 64 * s;
    v[s] = (e < E) ? l[e] : -INFINITY;
  }
  // selection j is kept by lane (j mod 64) in slot j / 64
  int sel_e[SLOTS];
  float sel_v[SLOTS];
  float top0 = 0.0f;
  uint32_t taken = 0;  // bit s set: v[s] of this lane already selected
  for (int j = 0; j < k; ++j) {
    // local best among untaken entries (ties: smaller e, i.e. smaller s)
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
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
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (j == lane + 64 * s) {
        sel_e[s] = be;
        sel_v[s] = bv;
      }
  }
  double u[SLOTS];
  double part = 0.0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    u[s] = 0.0;
    if (lane + 64 * s < k) {
      u[s] = exp(static_cast<double>(sel_v[s]) - static_cast<double>(top0));
      part += u[s];
    }
  }
  const double sum = wave_sum(part);
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    int j = lane + 64 * s;
    if (j < k) {
      out_ids[j] = sel_e[s];
      out_w[j] = static_cast<float>(u[s] / sum);
    }
  }
}

// One wavefront per token; SLOTS = the logits each lane holds (E <= 64 SLOTS).
template <int SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int T,
                                                   int E, int k) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_row<SLOTS>(logits + static_cast<size_t>(t) * E, E, k, ids + static_cast<size_t>(t) * k,
                  w + static_cast<size_t>(t) * k, threadIdx.x & 63);
}

// (value, index) a ranks before (value, index) b: larger logit first, equal
// logits by lower expert index.
__device__ __forceinline__ bool gate_before(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// Top-k (k <= min(G, 8)) of one token's E logits row[0..E) by G consecutive
// lanes (G = 4 or 8): each lane keeps its own sorted list of the 8 best of
// experts part, part + G, ... (a compare-exchange chain per expert), the G
// lists are merged pairwise (the 8 best of two sorted lists are the larger
// of a_i and b_{7-i}, a bitonic sequence that three half-cleaner stages
// sort), and lane j < k writes selection j with weight
// exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0) in fp64, the sum in i order.
template <int G>
__device__ __forceinline__ void topk_group(const float* row, int E, int k, int32_t* out_ids,
                                           float* out_w, int part, int lane) {
  float lv[8];
  int le[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    lv[p] = -INFINITY;
    le[p] = 0x7fffffff;
  }
  for (int e = part; e < E; e += G) {
    float xv = row[e];
    int xe = e;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (gate_before(xv, xe, lv[p], le[p])) {
        const float tv = lv[p];
        const int te = le[p];
        lv[p] = xv;
        le[p] = xe;
        xv = tv;
        xe = te;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < G; o <<= 1) {
    float ov[8];
    int oe[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      ov[p] = __shfl_xor(lv[p], o, 64);
      oe[p] = __shfl_xor(le[p], o, 64);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (gate_before(ov[7 - i], oe[7 - i], lv[i], le[i])) {
        lv[i] = ov[7 - i];
        le[i] = oe[7 - i];
      }
#pragma unroll
    for (int dist = 4; dist > 0; dist >>= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i & dist) == 0 && gate_before(lv[i + dist], le[i + dist], lv[i], le[i])) {
          const float tv = lv[i];
          const int te = le[i];
          lv[i] = lv[i + dist];
          le[i] = le[i + dist];
          lv[i + dist] = tv;
          le[i + dist] = te;
        }
  }
  float mv = lv[0];
  int me = le[0];
#pragma unroll
  for (int p = 1; p < 8; ++p)
    if (part == p) {
      mv = lv[p];
      me = le[p];
    }
  const double u = exp(static_cast<double>(mv) - static_cast<double>(lv[0]));
  const int base = lane - part;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += __shfl(u, base + j, 64);
  if (part < k) {
    out_ids[part] = me;
    out_w[part] = static_cast<float>(u / sum);
  }
}

// Router logits on the fp32 MFMA.  v_mfma_f32_16x16x4_f32 adds its four
// products to the accumulator as four sequential fused multiply-adds, k = 0..3
// in order (measured bit for bit on gfx950 against fmaf over 5 million
// outputs, mixed magnitudes and subnormals), so a chain of these MFMAs over
// hidden steps of four, ascending, is exactly the fixed fma order of every
// logit.  Lane group lg of an operand therefore holds hidden index 4s + lg of
// step s.
//
// Workgroup: 16 TG tokens x 16 TEF experts, TG WS waves; wave w owns tokens
// 16 (w % TG).. and TEF / WS fragments of 16 experts (the weight fragment is
// MFMA operand A, so the accumulator is D[expert][token]: lane l holds experts
// 4(l/16) + r of token l % 16).  Chunks of KB hidden elements are staged in
// LDS as fp32, double-buffered: x rows as four groups (i mod 4) of KB/4
// consecutive steps, so a lane reads four steps of its token with one 16-byte
// load; gate_w in its own [i][e] order (row stride = 16 banks mod 32, so the
// four lane groups' rows never collide).  The next chunk's global loads are
// in flight while a chunk is multiplied.  With FUSE (one workgroup covers all
// E <= 256 experts) the workgroup then runs the top-k of its 64 tokens.
constexpr int kGateGroupPad = 4;  // floats of padding per x step group (LDS banks)

template <int TEF, int KB, int TG>
struct GateLds {
  static constexpr int GS = KB / 4 + kGateGroupPad;  // floats per x step group
  static constexpr int LDR = 4 * GS + 4;             // floats per staged x row
  static constexpr int WE = 16 * TEF + 16;           // floats per staged gate_w row
  static constexpr int BUF = 16 * TG * LDR + KB * WE;  // floats per buffer
};

// Activation quantisation fused into the gate's pass over x (QUANT 1: FP8
// E4M3 per 1x128 group with an fp32 scale amax / 448; QUANT 2: OCP MX FP8,
// E4M3 with an E8M0 scale per block of 32), the activation format of the FP8
// and MXFP4 expert GEMMs: the SFA load role of the MegaMoE-vs-MoE-systems
// page, section 2.1, fed without a second read of x.
struct GateQuant {
  uint8_t* q;         // [T][d] codes
  void* s;            // FP8: fp32 [T][s_stride]; MX: E8M0 bytes [T][d / 32]
  int64_t s_stride;   // FP8: floats per scale row
};

template <int TEF, int WS, int KB, int TG, bool BF16, bool FUSE, int QUANT>
__global__ __launch_bounds__(64 * TG * WS) void gate_kernel(const void* __restrict__ xv,
                                                        const void* __restrict__ wv,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ wts, int T, int d,
                                                        int E, int k, GateQuant gq) {
  using GL = GateLds<TEF, KB, TG>;
  constexpr int GS = GL::GS, LDR = GL::LDR, WE = GL::WE, BUF = GL::BUF;
  constexpr int NT = 64 * TG * WS;                   // threads
  constexpr int XROWS = 16 * TG, WROWS = 16 * TEF, FPW = TEF / WS;
  constexpr int EPC = BF16 ? 8 : 4;                  // elements per 16-byte load
  constexpr int XCH = XROWS * (KB / EPC), WCH = KB * (WROWS / EPC);
  constexpr int XR = (XCH + NT - 1) / NT, WR = (WCH + NT - 1) / NT;
  static_assert(KB % 32 == 0 && WROWS % EPC == 0 && TEF % WS == 0, "chunk shape");
  extern __shared__ __attribute__((aligned(16))) float gate_lds[];  // [2][BUF]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int tg = wave % TG, fr0 = (wave / TG) * FPW;  // token group, first fragment
  const int t0 = blockIdx.x * XROWS, e0 = blockIdx.y * WROWS;

  u32x4 xr[XR], wr[WR];
  bool wvec[WR];
  // raw 16-byte piece r of chunk i0 (zero outside x / gate_w)
  auto load_x = [&](int i0, int r) {
    const int idx = tid + NT * r;
    const int tl = idx / (KB / EPC), il = (idx % (KB / EPC)) * EPC;
    const int t = t0 + tl, i = i0 + il;
    xr[r] = u32x4{0u, 0u, 0u, 0u};
    if (idx < XCH && t < T && i < d) {
      const size_t o = static_cast<size_t>(t) * d + i;
      xr[r] = BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(xv) + o)
                   : *reinterpret_cast<const u32x4*>(static_cast<const float*>(xv) + o);
    }
  };
  auto load_w = [&](int i0, int r) {
    const int idx = tid + NT * r;
    const int il = idx / (WROWS / EPC), el = (idx % (WROWS / EPC)) * EPC;
    const int e = e0 + el, i = i0 + il;
    wr[r] = u32x4{0u, 0u, 0u, 0u};
    wvec[r] = idx < WCH && i < d && E % EPC == 0 && e + EPC <= E;
    if (wvec[r]) {
      const size_t o = static_cast<size_t>(i) * E + e;
      wr[r] = BF16 ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(wv) + o)
                   : *reinterpret_cast<const u32x4*>(static_cast<const float*>(wv) + o);
    }
  };
  // widen piece r to fp32 and store it into buffer b
  auto store_x = [&](int b, int r) {
    float* Lx = gate_lds + b * BUF;
    const int idx = tid + NT * r;
    if (idx < XCH) {
      const int tl = idx / (KB / EPC), il = (idx % (KB / EPC)) * EPC;
      float v[EPC];
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = __uint_as_float(xr[r][q] << 16);
          v[2 * q + 1] = __uint_as_float(xr[r][q] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < EPC; ++q) v[q] = __uint_as_float(xr[r][q]);
      }
      float* row = Lx + tl * LDR;  // element i of the chunk at group i % 4, step i / 4
#pragma unroll
      for (int q = 0; q < EPC; ++q) row[q % 4 * GS + (il + q) / 4] = v[q];
    }
  };
  auto store_w = [&](int b, int i0, int r) {
    float* Lw = gate_lds + b * BUF + XROWS * LDR;
    const int idx = tid + NT * r;
    if (idx < WCH) {
      const int il = idx / (WROWS / EPC), el = (idx % (WROWS / EPC)) * EPC;
      const int i = i0 + il;
      float v[EPC];
      if (wvec[r]) {
        if (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(wr[r][q] << 16);
            v[2 * q + 1] = __uint_as_float(wr[r][q] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int q = 0; q < EPC; ++q) v[q] = __uint_as_float(wr[r][q]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int eq = e0 + el + q;
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
      for (int q = 0; q < EPC; q += 4)
        *reinterpret_cast<f32x4*>(Lw + il * WE + el + q) =
            f32x4{v[q], v[q + 1], v[q + 2], v[q + 3]};
    }
  };
  // Fused quantisation of x piece r of chunk i0 (still raw in xr[r]).  The
  // KB / EPC lanes that hold one token's part of a chunk are consecutive
  // lanes of one wave, and a thread holds the same (token, column) piece in
  // every chunk.  MX: a block of 32 is four of those lanes, so it is
  // encoded at once.  FP8: the thread keeps its raw pieces of the current
  // 128-column group and their running amax; when the chunk that ends the
  // group is staged, the lanes of the token combine their maxima and each
  // thread encodes its pieces.  Called in wave-uniform control flow (the
  // shuffles).
  static_assert(QUANT == 0 || (BF16 && 128 % KB == 0), "quantised activations are bf16");
  constexpr int QPIECES = (QUANT == 1) ? 128 / KB : 1;  // a thread's pieces of one group
  float qmax[XR];
  u32x4 qraw[XR][QPIECES];  // FP8: the raw pieces of the current group
#pragma unroll
  for (int r = 0; r < XR; ++r) qmax[r] = 0.f;
  auto quant_piece = [&](int i0, int r) {
    const int idx = tid + NT * r;
    const int tl = idx / (KB / EPC), il = (idx % (KB / EPC)) * EPC;
    const int t = t0 + tl, i = i0 + il;
    // (when the experts are split over several workgroup columns, all of
    // them read the same x rows: 128-column group g is written by column
    // g mod gridDim.y, which spreads the encoding over the columns when
    // there are few token rows)
    const bool writer = blockIdx.y == static_cast<unsigned>(i0 / 128) % gridDim.y;
    const bool valid = idx < XCH && t < T && i < d;
    float v[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = valid ? __uint_as_float(xr[r][q] << 16) : 0.f;
      v[2 * q + 1] = valid ? __uint_as_float(xr[r][q] & 0xffff0000u) : 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
    if constexpr (QUANT == 2) {
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      const int xe = mx_exponent_e4m3(m);
      if (valid && writer) {
        u32x2 c;
        c.x = f32x4_to_e4m3x4(__builtin_ldexpf(v[0], -xe), __builtin_ldexpf(v[1], -xe),
                              __builtin_ldexpf(v[2], -xe), __builtin_ldexpf(v[3], -xe));
        c.y = f32x4_to_e4m3x4(__builtin_ldexpf(v[4], -xe), __builtin_ldexpf(v[5], -xe),
                              __builtin_ldexpf(v[6], -xe), __builtin_ldexpf(v[7], -xe));
        *reinterpret_cast<u32x2*>(gq.q + static_cast<size_t>(t) * d + i) = c;
        if ((il & 31) == 0)
          static_cast<uint8_t*>(gq.s)[static_cast<size_t>(t) * (d / 32) + i / 32] =
              static_cast<uint8_t>(xe + 127);
      }
    } else if constexpr (QUANT == 1) {
      qmax[r] = fmaxf(qmax[r], m);
      qraw[r][(i0 % 128) / KB] = xr[r];
      if ((i0 + KB) % 128 == 0) {  // this chunk ends a 128-column group
        float a = qmax[r];
#pragma unroll
        for (int o = 1; o < KB / EPC; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
        qmax[r] = 0.f;
        const float sc = (a == 0.f) ? 1.0f : __fdiv_rn(a, 448.0f);
        const int g0 = i0 + KB - 128;
        if (idx < XCH && t < T && writer) {
#pragma unroll
          for (int c = 0; c < 128 / KB; ++c) {
            const int col = g0 + c * KB + il;
            const u32x4 raw = qraw[r][c];
            // (x / sc with the IEEE division: these codes are the stated
            // recipe's, bit for bit)
            float v8[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v8[2 * q] = __fdiv_rn(__uint_as_float(raw[q] << 16), sc);
              v8[2 * q + 1] = __fdiv_rn(__uint_as_float(raw[q] & 0xffff0000u), sc);
            }
            u32x2 cd;
            cd.x = f32x4_to_e4m3x4(v8[0], v8[1], v8[2], v8[3]);
            cd.y = f32x4_to_e4m3x4(v8[4], v8[5], v8[6], v8[7]);
            *reinterpret_cast<u32x2*>(gq.q + static_cast<size_t>(t) * d + col) = cd;
          }
          if (il == 0) static_cast<float*>(gq.s)[static_cast<size_t>(t) * gq.s_stride + g0 / 128] = sc;
        }
      }
    }
  };

  // piece p of the staging (x pieces, then gate_w pieces): store the loaded
  // piece of chunk i0 into buffer b, then (if i2 < d) load the same piece of
  // chunk i2 into the registers it frees
  constexpr int NP = XR + WR;
  auto stage = [&](int p, int b, int i0, int i2) {
    if (p < XR) {
      if constexpr (QUANT != 0) quant_piece(i0, p);
      store_x(b, p);
      if (i2 < d) load_x(i2, p);
    } else {
      store_w(b, i0, p - XR);
      if (i2 < d) load_w(i2, p - XR);
    }
  };

  f32x4 acc[FPW];
#pragma unroll
  for (int f = 0; f < FPW; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the MFMA chain over chunk i0 in buffer b, four steps at a time.  With up
  // to four fragments per wave, the LDS operands of the next four steps are
  // read before the MFMAs of the current ones, so their latency hides behind
  // the chain, and when the chunk is full and another follows, the staging
  // of chunk i0 + KB into buffer b ^ 1 (with the loads of chunk i0 + 2 KB) is
  // spread over the chain, one piece after each four steps, where it issues
  // while the next MFMA waits for the previous result.  Eight fragments
  // (eight independent chains per wave) have no registers for a second
  // operand set; their staging follows the chain.
  struct Ops {
    f32x4 x;
    float w[4][FPW];
  };
  auto compute = [&](int b, int i0, bool staged) {
    const int i2 = i0 + 2 * KB;  // chunk loaded into the registers staging frees
    const float* Lx = gate_lds + b * BUF;
    const float* xrow = Lx + (16 * tg + l16) * LDR + lg * GS;
    const float* wcol = Lx + XROWS * LDR + lg * WE + 16 * fr0 + l16;  // row 4s + lg
    auto ops = [&](int s, Ops& o) {
      o.x = *reinterpret_cast<const f32x4*>(xrow + s);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int f = 0; f < FPW; ++f) o.w[u][f] = wcol[4 * (s + u) * WE + 16 * f];
    };
    auto mm = [&](const Ops& o) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int f = 0; f < FPW; ++f)
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.w[u][f], o.x[u], acc[f], 0, 0, 0);
    };
    Ops o0, o1;
    if (FPW >= 8) {  // two operand sets would not fit in the registers
      const int steps = min(KB, d - i0) / 4;
      for (int s = 0; s < steps; s += 4) {
        ops(s, o0);
        mm(o0);
      }
      if (staged) {
#pragma unroll
        for (int p = 0; p < NP; ++p) stage(p, b ^ 1, i0 + KB, i2);
      }
      return;
    }
    ops(0, o0);
    if (staged) {
      constexpr int NI = KB / 16;  // groups of four steps in a full chunk (even)
#pragma unroll
      for (int it = 0; it < NI; it += 2) {
        ops(4 * it + 4, o1);
        mm(o0);
        if (it < NP) stage(it, b ^ 1, i0 + KB, i2);
        if (it + 2 < NI) ops(4 * it + 8, o0);
        mm(o1);
        if (it + 1 < NP) stage(it + 1, b ^ 1, i0 + KB, i2);
      }
#pragma unroll
      for (int p = NI; p < NP; ++p) stage(p, b ^ 1, i0 + KB, i2);
    } else {
      const int steps = min(KB, d - i0) / 4;  // d % 32 == 0: a multiple of 8
      for (int s = 0; s < steps; s += 8) {
        ops(s + 4, o1);
        mm(o0);
        if (s + 8 < steps) ops(s + 8, o0);
        mm(o1);
      }
    }
  };

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p < XR) load_x(0, p);
    else load_w(0, p - XR);
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) stage(p, 0, 0, KB);
  __syncthreads();
  int buf = 0;
  for (int i0 = 0; i0 < d; i0 += KB) {
    compute(buf, i0, i0 + KB < d);
    __syncthreads();
    buf ^= 1;
  }

  // logits (+ bias, one fp32 add) of this wave's 16 tokens x 16 FPW experts
  const int t = t0 + 16 * tg + l16;
  float* tile = gate_lds;  // FUSE: [16 TG][E + 1] logits of the workgroup
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + 16 * (fr0 + f) + 4 * lg + r;
      if (e < E) {
        float l = acc[f][r];
        if (bias) l = l + bias[e];
        if (t < T) logits[static_cast<size_t>(t) * E + e] = l;
        if (FUSE) tile[(16 * tg + l16) * (E + 1) + e] = l;
      }
    }
  }
  if constexpr (FUSE) {
    // top-k of the workgroup's tokens, 4 WS consecutive lanes per token
    constexpr int G = 4 * WS;
    __syncthreads();
    const int row = tid / G, tj = t0 + row;
    if (tj < T)
      topk_group<G>(tile + row * (E + 1), E, k, ids + static_cast<size_t>(tj) * k,
                    wts + static_cast<size_t>(tj) * k, tid % G, lane);
  }
}

// Raise the dynamic LDS limit of one gate_kernel instantiation to the 160 KB
// of a CU, once per instantiation (a function-local static of a template is
// per instantiation); the result of that first call is returned every time.
template <int TEF, int WS, int KB, int TG, bool BF16, bool FUSE, int QUANT>
hipError_t gate_lds_attr() {
  static const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gate_kernel<TEF, WS, KB, TG, BF16, FUSE, QUANT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  return e;
}

template <int TEF, int WS, int KB, int TG, bool BF16, bool FUSE, int QUANT>
int launch_gate_variant(const void* x, const void* gate_w, const float* bias, float* logits,
                        int32_t* ids, float* w, int T, int d, int E, int k, GateQuant gq,
                        hipStream_t s) {
  const hipError_t attr = gate_lds_attr<TEF, WS, KB, TG, BF16, FUSE, QUANT>();
  if (attr != hipSuccess) return static_cast<int>(attr);
  const dim3 grid((T + 16 * TG - 1) / (16 * TG), FUSE ? 1 : (E + 16 * TEF - 1) / (16 * TEF));
  size_t lds = sizeof(float) * 2 * static_cast<size_t>(GateLds<TEF, KB, TG>::BUF);
  if (FUSE) lds = std::max(lds, sizeof(float) * 16 * TG * static_cast<size_t>(E + 1));
  gate_kernel<TEF, WS, KB, TG, BF16, FUSE, QUANT>
      <<<grid, 64 * TG * WS, lds, s>>>(x, gate_w, bias, logits, ids, w, T, d, E, k, gq);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

void launch_topk(const float* logits, int32_t* ids, float* w, int T, int E, int k,
                 hipStream_t s) {
  const dim3 grid((T + 3) / 4);
  if (E <= 64) topk_kernel<1><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
  else if (E <= 128) topk_kernel<2><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
  else if (E <= 256) topk_kernel<4><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
  else if (E <= 512) topk_kernel<8><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
  else topk_kernel<16><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
}

// Gate: logits on the MFMA, then top-k -- inside the same workgroup when one
// workgroup covers every expert (E <= 256), k <= 8 and the tokens alone give
// the chip >= 1024 waves; otherwise experts are split across workgroups (as many
// fragments per wave as still give >= 1024 waves) and a top-k kernel follows.
// Two waves share each token group where the fragments allow, so that one
// wave's staging overlaps the other's MFMAs.  d % 32 == 0.  Returns a
// hipError_t (hipSuccess when everything was enqueued).
int launch_gate(const void* x, const void* gate_w, const float* bias, float* logits,
                int32_t* ids, float* w, int T, int d, int E, int k, bool bf16, hipStream_t s,
                int quant, uint8_t* xq, void* xs, int64_t xs_stride) {
  if (T <= 0) return 0;
  const long long tw = (T + 15) / 16;  // token waves
  const int ef = (E + 15) / 16;        // expert fragments
  int tef = 1;
  bool fuse = ef <= 16 && tw >= 1024 && k <= 8;
  if (fuse) {
    tef = ef <= 1 ? 1 : ef <= 2 ? 2 : ef <= 4 ? 4 : ef <= 8 ? 8 : 16;
    if (tef == 1 && k > 4) fuse = false;  // 4 lanes per token with one wave per group
  }
  if (!fuse) {
    tef = 1;
    for (int c : {4, 2}) {
      if (c <= ef && tw * ((ef + c - 1) / c) >= 1024) {
        tef = c;
        break;
      }
    }
  }
  // fused quantisation: bf16 activations only (FP8 and MXFP4 layers)
  if (quant != 0 && !bf16) return static_cast<int>(hipErrorInvalidValue);
  const GateQuant gq{xq, xs, xs_stride};
  int rc = -1;
  // (TEF, WS, KB, TG): the widest expert tiles stage 128 tokens per
  // workgroup, which halves the gate_w traffic per token
#define MOE_GQ(TEF_, WS_, KB_, TG_, FU_, Q_)                                                  \
  rc = launch_gate_variant<TEF_, WS_, KB_, TG_, true, FU_, Q_>(x, gate_w, bias, logits, ids, w, \
                                                              T, d, E, k, gq, s)
#define MOE_G(TEF_, WS_, KB_, TG_)                                                            \
  if (tef == TEF_) {                                                                          \
    if (!bf16) {                                                                              \
      if (fuse)                                                                               \
        rc = launch_gate_variant<TEF_, WS_, KB_, TG_, false, true, 0>(                        \
            x, gate_w, bias, logits, ids, w, T, d, E, k, gq, s);                              \
      else                                                                                    \
        rc = launch_gate_variant<TEF_, WS_, KB_, TG_, false, false, 0>(                       \
            x, gate_w, bias, logits, ids, w, T, d, E, k, gq, s);                              \
    } else if (fuse) {                                                                        \
      if (quant == 1) MOE_GQ(TEF_, WS_, KB_, TG_, true, 1);                                   \
      else if (quant == 2) MOE_GQ(TEF_, WS_, KB_, TG_, true, 2);                              \
      else MOE_GQ(TEF_, WS_, KB_, TG_, true, 0);                                              \
    } else {                                                                                  \
      if (quant == 1) MOE_GQ(TEF_, WS_, KB_, TG_, false, 1);                                  \
      else if (quant == 2) MOE_GQ(TEF_, WS_, KB_, TG_, false, 2);                             \
      else MOE_GQ(TEF_, WS_, KB_, TG_, false, 0);                                             \
    }                                                                                         \
  }
  MOE_G(1, 1, 128, 4)
  MOE_G(2, 2, 128, 4)
  MOE_G(4, 2, 64, 4)
  MOE_G(8, 2, 64, 4)
  MOE_G(16, 2, 32, 8)
#undef MOE_G
#undef MOE_GQ
  if (rc != 0) return rc;
  if (!fuse) launch_topk(logits, ids, w, T, E, k, s);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
