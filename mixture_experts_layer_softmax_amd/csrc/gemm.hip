// gemm.hip -- persistent grouped expert GEMMs on CDNA4 MFMA.
//
// Phase 1 (W1/W3 + SwiGLU): for every m-tile of one expert's slots, the
// activation rows are gathered straight from x (or its FP8 codes) into LDS
// by the slot -> token index -- no permuted copy of x exists in memory (the
// ScatterMoE step of the lineage on the MegaMoE-vs-MoE-systems page, section
// 1) -- and multiplied with the gate (W1) and up (W3) weights of the expert.
// Gate and up columns of the same f index land in the same lane, so SwiGLU
// is applied in registers and h is rounded once to the activation format
// (bf16 RNE, fp32, or FP8 with a fresh 1x128 scale: the epilogue role
// "SwiGLU + amax + quantise" on that page, section 2.1).
// Phase 2 (W2): h rows of an m-tile times the expert's down weights, fp32 Y.
//
// Scheduling: a persistent grid sized from occupancy pulls (m-tile, n-tile)
// tasks from an integer atomic counter -- a work-conserving device-side tile
// queue (FlashMoE Kernel page, Architecture: the scheduler hands out work by
// readiness; MegaMoE-vs-MoE-systems page, section 2.7: a global atomic task
// counter).  Skewed experts simply own more tasks; idle CUs keep pulling.
// Padding rows exist only inside the last m-tile of an expert and are never
// stored (FlashMoE Kernel page, Communication: padding is local, just before
// compute).
//
// MFMA mapping: the weight fragment is the MFMA "A" operand and the token
// fragment the "B" operand, so the 16x16 result tile is D[n][slot]: lane l
// holds n = 4*(l/16) + r (r = 0..3) of slot l%16 -- four consecutive output
// columns of one row, which makes every epilogue store a 8- or 16-byte
// vector and puts gate/up pairs in the same lane.
// LDS rows are 128 bytes of K (64 bf16, 32 fp32 or 128 fp8) split in eight
// 16-byte chunks stored XOR-swizzled by (row & 7).
#include "device_common.hpp"
#include "launch.hpp"

#include <cstdlib>
#include <mutex>

namespace moe {

namespace {

constexpr int kRowBytes = 128;

template <int DT>
struct ESize;
template <>
struct ESize<kF32> { static constexpr int v = 4; };
template <>
struct ESize<kBF16> { static constexpr int v = 2; };
template <>
struct ESize<kFP8> { static constexpr int v = 1; };

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// Bytes of LDS shared by the main-loop stages and the epilogue staging.
template <int DT, int PHASE, int BM, int BN, int WM>
struct StageBytes {
  static constexpr int main_loop = 2 * (BM + BN) * kRowBytes;
  static constexpr int epilogue = (BM / WM) * ((PHASE == 1) ? BN / 2 : BN) *
                                  ((PHASE == 1) ? ESize<DT>::v : 4);
  static constexpr int v = main_loop > epilogue ? main_loop : epilogue;
};

template <int DT, int PHASE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int kThreads = WM * WN * 64;
  constexpr int ES = ESize<DT>::v;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int ACH = BM * 8, BCH = BN * 8;  // 16-byte chunks per K-step
  constexpr int RA = (ACH + kThreads - 1) / kThreads;
  constexpr int RB = (BCH + kThreads - 1) / kThreads;
  static_assert(WM * WN == 4 || WM * WN == 8, "four or eight waves");
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(PHASE == 2 || TN % 2 == 0, "gate/up pairs");
  static_assert(!(DT == kFP8 && PHASE == 1) || BN == 256, "FP8 h groups of 128 f");

  // LDS: the two K-step stages of A and B, reused by the epilogue staging,
  // then (FP8 phase 1) the per-wave row maxima
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* As = lds;                                  // [2][BM][128]
  uint8_t* Bs = lds + 2 * BM * kRowBytes;             // [2][BN][128]
  float* red = reinterpret_cast<float*>(lds + StageBytes<DT, PHASE, BM, BN, WM>::v);  // [WN][BM]
  __shared__ int s_task;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t K = g.K, N = g.N;
  const int ksteps = static_cast<int>(K * ES / kRowBytes);
  const int kblocks = static_cast<int>(K / 128);  // FP8 scale blocks along K
  const int nblocks = static_cast<int>(N / 128);
  // XCD-aware work queue.  Workgroups of a persistent launch are dealt to the
  // eight XCDs round-robin, so workgroup b runs on XCD b % 8 and shares that
  // XCD's L2 with the others there.  The m-tiles are cut into chunks of kGM
  // consecutive m-tiles; chunk c belongs to XCD c % 8, whose workgroups take
  // its tasks n-tile by n-tile (kGM m-tiles x n-tiles in flight per XCD:
  // activation rows reused across n-tiles and weight rows across m-tiles in
  // one L2).  A drained XCD queue makes its workgroups steal from the others,
  // so the queue stays work-conserving under routing skew.
  constexpr int kXcd = 8, kGM = 4;
  const int M = *g.tm.n_mtiles, NT = g.n_tiles_n;
  const int nchunks = (M + kGM - 1) / kGM;
  const int chunk_tasks = kGM * NT;
  const int xcd = static_cast<int>(blockIdx.x) % kXcd;
  int* queue = g.tm.queue + kXcd * g.queue_idx;

  for (;;) {
    if (tid == 0) {
      int task = -1;
      for (int s = 0; s < kXcd && task < 0; ++s) {
        const int y = (xcd + s) % kXcd;
        const int owned = nchunks > y ? (nchunks - y + kXcd - 1) / kXcd : 0;
        const int limit = owned * chunk_tasks;
        for (;;) {
          if (__hip_atomic_load(&queue[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= limit)
            break;
          const int v = atomicAdd(&queue[y], 1);
          if (v >= limit) break;
          const int p = v % chunk_tasks;
          const int mt = (y + kXcd * (v / chunk_tasks)) * kGM + p % kGM;
          if (mt < M) {  // the last chunk may hold fewer than kGM m-tiles
            task = mt * NT + p / kGM;
            break;
          }
        }
      }
      s_task = task;
    }
    __syncthreads();
    const int task = s_task;
    if (task < 0) break;
    const int mt = task / g.n_tiles_n;
    const int nt = task - mt * g.n_tiles_n;
    const int e = g.tm.e[mt], row0 = g.tm.row0[mt], rows = g.tm.rows[mt];
    const int64_t n0 = static_cast<int64_t>(nt) * BN;

    // ---- source of every 16-byte chunk this thread stages: 32-bit byte
    // offsets from wave-uniform bases (the host checks that every operand
    // spans less than 2^31 bytes per expert) ----
    const int64_t w_bytes = N * K * ES;  // one expert's weight matrix
    const uint8_t* b0 = g.B0 + static_cast<int64_t>(e) * w_bytes;
    const uint8_t* b1 = (PHASE == 1) ? g.B1 + static_cast<int64_t>(e) * w_bytes : b0;
    uint32_t oa[RA], ob[RB];
    uint32_t up_mask = 0;  // bit j: chunk j of B comes from the up (W3) matrix
#pragma unroll
    for (int j = 0; j < RA; ++j) {
      const int ci = tid + kThreads * j;
      const int r = min(ci >> 3, rows - 1);  // padding rows re-read a valid row
      const int64_t src = g.gather ? g.gather[row0 + r] : static_cast<int64_t>(row0 + r);
      oa[j] = static_cast<uint32_t>(src * g.a_row_bytes + (ci & 7) * 16);
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int ci = tid + kThreads * j;
      const int64_t n = n0 + (ci >> 3);
      int64_t col;
      if (PHASE == 1) {  // combined rows: 16 gate rows, then 16 up rows, per f block
        col = (n >> 5) * 16 + (n & 15);
        if (n & 16) up_mask |= 1u << j;
      } else {
        col = n;
      }
      col = min(col, N - 1);
      ob[j] = static_cast<uint32_t>(col * K * ES + (ci & 7) * 16);
    }

    // Prefetch registers of the next K-step.  Written with plain loops (no
    // lambdas capturing the arrays by reference), so they stay in VGPRs.
    u32x4 ra[RA], rb[RB];
#define MOE_GLOAD(KS)                                                                   \
  do {                                                                                  \
    const uint32_t off_ = static_cast<uint32_t>(KS) * kRowBytes;                        \
    _Pragma("unroll") for (int j = 0; j < RA; ++j) if (ACH % kThreads == 0 ||            \
                                                        tid + kThreads * j < ACH)       \
        ra[j] = *reinterpret_cast<const u32x4*>(g.A + (oa[j] + off_));                  \
    _Pragma("unroll") for (int j = 0; j < RB; ++j) if (BCH % kThreads == 0 ||            \
                                                        tid + kThreads * j < BCH)       \
        rb[j] = *reinterpret_cast<const u32x4*>(((up_mask >> j) & 1u ? b1 : b0) +       \
                                                (ob[j] + off_));                        \
  } while (0)
#define MOE_LSTORE(BUF)                                                                 \
  do {                                                                                  \
    _Pragma("unroll") for (int j = 0; j < RA; ++j) {                                    \
      const int ci = tid + kThreads * j;                                                \
      if (ACH % kThreads == 0 || ci < ACH)                                              \
        *reinterpret_cast<u32x4*>(As + (BUF) * BM * kRowBytes + swz(ci >> 3, ci & 7)) = \
            ra[j];                                                                      \
    }                                                                                   \
    _Pragma("unroll") for (int j = 0; j < RB; ++j) {                                    \
      const int ci = tid + kThreads * j;                                                \
      if (BCH % kThreads == 0 || ci < BCH)                                              \
        *reinterpret_cast<u32x4*>(Bs + (BUF) * BN * kRowBytes + swz(ci >> 3, ci & 7)) = \
            rb[j];                                                                      \
    }                                                                                   \
  } while (0)

    // FP8: per token fragment i, the A-scale row offset of the lane's slot
    uint32_t sa_off[TM];
    if constexpr (DT == kFP8) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = min(wm * WTM + 16 * i + l16, rows - 1);
        const int64_t src = g.gather ? g.gather[row0 + r] : static_cast<int64_t>(row0 + r);
        sa_off[i] = static_cast<uint32_t>(src * kblocks);
      }
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < ksteps) MOE_GLOAD(ks + 1);
      const uint8_t* Ab = As + cur * BM * kRowBytes;
      const uint8_t* Bb = Bs + cur * BN * kRowBytes;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 wf[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wf[j] = *reinterpret_cast<const bf16x8*>(Bb + swz(wn * WTN + 16 * j + l16, kk * 4 + lg));
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (wm * WTM + 16 * i >= rows) break;  // padding rows only: wave-uniform
            const bf16x8 xf =
                *reinterpret_cast<const bf16x8*>(Ab + swz(wm * WTM + 16 * i + l16, kk * 4 + lg));
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf, acc[i][j], 0, 0, 0);
          }
        }
      } else if constexpr (DT == kF32) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          f32x4 wf[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wf[j] = *reinterpret_cast<const f32x4*>(Bb + swz(wn * WTN + 16 * j + l16, kk * 4 + lg));
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (wm * WTM + 16 * i >= rows) break;
            const f32x4 xf =
                *reinterpret_cast<const f32x4*>(Ab + swz(wm * WTM + 16 * i + l16, kk * 4 + lg));
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[j][u], xf[u], acc[i][j], 0, 0, 0);
          }
        }
      } else {  // FP8: one 16x16x128 MFMA per fragment pair and K block
        i32x8 wf[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = wn * WTN + 16 * j + l16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(Bb + swz(r, 2 * lg));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(Bb + swz(r, 2 * lg + 1));
          wf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        float s_b0, s_b1 = 0.f;
        if (PHASE == 1) {
          const int fb = static_cast<int>(n0 / 256);  // 128 f columns per workgroup tile
          s_b0 = g.sb0[(static_cast<int64_t>(e) * kblocks + ks) * nblocks + fb];
          s_b1 = g.sb1[(static_cast<int64_t>(e) * kblocks + ks) * nblocks + fb];
        } else {
          const int nb = static_cast<int>((n0 + wn * WTN) / 128);
          s_b0 = g.sb0[(static_cast<int64_t>(e) * kblocks + ks) * nblocks + nb];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (wm * WTM + 16 * i >= rows) break;  // padding rows only: wave-uniform
          const int r = wm * WTM + 16 * i + l16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(Ab + swz(r, 2 * lg));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(Ab + swz(r, 2 * lg + 1));
          const i32x8 xf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const float s_a = g.sa[sa_off[i] + ks];
          const float sg = s_a * s_b0, su = s_a * s_b1;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, z, 0, 0,
                                                                              0, 127, 0, 127);
            const float sc = (PHASE == 1 && (j & 1)) ? su : sg;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(p[q], sc, acc[i][j][q]);
          }
          // keep each fragment's MFMAs next to their rescale: hoisting all of
          // them would hold TM x TN fresh results live and spill
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (ks + 1 < ksteps) MOE_LSTORE(cur ^ 1);
      __syncthreads();
    }

#undef MOE_GLOAD
#undef MOE_LSTORE

    // ---------------- epilogue ----------------
    // Output values are staged in LDS (free after the main loop's last
    // barrier) so that every global store is a 16-byte piece of a contiguous
    // row segment; one pass per wave row wm.  Staged rows are XOR-swizzled by
    // 16-byte chunk to keep the fragment writes off a single bank group.
    constexpr int OUT_COLS = (PHASE == 1) ? BN / 2 : BN;
    constexpr int OUT_ES = (PHASE == 1) ? ES : 4;
    constexpr int ROWB = OUT_COLS * OUT_ES;
    constexpr int CPR = ROWB / 16;
    constexpr int XM = (CPR >= 16 ? 16 : CPR) - 1;
    uint8_t* stage = lds;
    auto st_off = [&](int r, int cbyte) {
      return r * ROWB + ((((cbyte >> 4) ^ (r & XM)) << 4) | (cbyte & 15));
    };
    const int64_t col0 = (PHASE == 1) ? n0 / 2 : n0;

    if constexpr (PHASE == 1 && DT == kFP8) {
      // h = SiLU(gate) * up in fp32 (in place), then the row amax over the
      // tile's 128 f columns: lanes, then the WN waves through LDS
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float m = 0.f;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[i][2 * p][r] = silu(acc[i][2 * p][r]) * acc[i][2 * p + 1][r];
            m = fmaxf(m, fabsf(acc[i][2 * p][r]));
          }
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (lg == 0) red[wn * BM + wm * WTM + 16 * i + l16] = m;
      }
      __syncthreads();
    }

    for (int pass = 0; pass < WM; ++pass) {
      if (wm == pass) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = 16 * i + l16;  // row within this pass
          if constexpr (PHASE == 2) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
              *reinterpret_cast<f32x4*>(stage + st_off(r, (wn * WTN + 16 * j + 4 * lg) * 4)) =
                  acc[i][j];
          } else if constexpr (DT == kFP8) {
            const int lr = pass * WTM + r;
            float amax = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red[w * BM + lr]);
            const float sc = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
#pragma unroll
            for (int p = 0; p < TN / 2; ++p) {
              uint32_t packed = 0;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                packed |= f32_to_e4m3(__fdiv_rn(acc[i][2 * p][q], sc)) << (8 * q);
              *reinterpret_cast<uint32_t*>(stage + st_off(r, wn * (WTN / 2) + 16 * p + 4 * lg)) =
                  packed;
            }
            if (wn == 0 && lg == 0 && lr < rows)
              g.sc[static_cast<int64_t>(row0 + lr) * (N / 128) + n0 / 256] = sc;
          } else {
#pragma unroll
            for (int p = 0; p < TN / 2; ++p) {
              float h[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) h[q] = silu(acc[i][2 * p][q]) * acc[i][2 * p + 1][q];
              const int cb = (wn * (WTN / 2) + 16 * p + 4 * lg) * ES;
              if constexpr (DT == kBF16) {
                u32x2 v;
                v.x = f32_to_bf16_rne(h[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(h[1])) << 16);
                v.y = f32_to_bf16_rne(h[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(h[3])) << 16);
                *reinterpret_cast<u32x2*>(stage + st_off(r, cb)) = v;
              } else {
                *reinterpret_cast<f32x4*>(stage + st_off(r, cb)) = f32x4{h[0], h[1], h[2], h[3]};
              }
            }
          }
        }
      }
      __syncthreads();
      for (int idx = tid; idx < WTM * CPR; idx += kThreads) {
        const int r = idx / CPR, c = idx - r * CPR;
        const int lr = pass * WTM + r;
        const int64_t col = col0 + c * (16 / OUT_ES);
        if (lr < rows && col < N)
          *reinterpret_cast<u32x4*>(g.C + (static_cast<int64_t>(row0 + lr) * N + col) * OUT_ES) =
              *reinterpret_cast<const u32x4*>(stage + r * ROWB + ((c ^ (r & XM)) << 4));
      }
      __syncthreads();
    }
  }
}

template <int DT, int PHASE, int BM, int BN, int WM, int WN>
struct Variant {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int lds_bytes() {
    return StageBytes<DT, PHASE, BM, BN, WM>::v + ((DT == kFP8 && PHASE == 1) ? WN * BM * 4 : 0);
  }
  static int launch(const GemmArgs& a, hipStream_t s) {
    auto kern = grouped_gemm_kernel<DT, PHASE, BM, BN, WM, WN>;
    static int grid = 0;
    static std::once_flag once;
    std::call_once(once, [&] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes());
      int dev = 0, cus = 0, per_cu = 0;
      (void)hipGetDevice(&dev);
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds_bytes());
      grid = max(1, cus) * max(1, per_cu);
    });
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds_bytes(), s, a);
    return static_cast<int>(hipGetLastError());
  }
  static constexpr int tile_n() { return BN; }
};

// Tuning selector: MOE_GEMM_VARIANT picks an alternative tile shape for the
// tile heights that have one (read once; 0 = default).
int variant_choice() {
  static int v = [] {
    const char* e = getenv("MOE_GEMM_VARIANT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Kernel variant per (dtype, phase, tile height, tuning variant).
template <typename F>
int dispatch_var(int phase, int dtype, int bm, int var, F&& f) {
#define MOE_V(DT, P, BM_, VAR, BN_, WM_, WN_)                     \
  if (dtype == DT && phase == P && bm == BM_ && var == VAR)        \
    return f(Variant<DT, P, BM_, BN_, WM_, WN_>{});
  MOE_V(kBF16, 1, 256, 0, 256, 2, 4)
  MOE_V(kBF16, 2, 256, 0, 256, 2, 4)
  MOE_V(kBF16, 1, 256, 1, 256, 2, 2)
  MOE_V(kBF16, 2, 256, 1, 256, 2, 2)
  MOE_V(kBF16, 1, 128, 0, 128, 2, 2)
  MOE_V(kBF16, 2, 128, 0, 128, 2, 2)
  MOE_V(kBF16, 1, 128, 1, 256, 1, 4)
  MOE_V(kBF16, 2, 128, 1, 256, 1, 4)
  MOE_V(kBF16, 1, 128, 2, 256, 2, 4)
  MOE_V(kBF16, 2, 128, 2, 256, 2, 4)
  MOE_V(kBF16, 1, 64, 0, 128, 1, 4)
  MOE_V(kBF16, 2, 64, 0, 128, 1, 4)
  MOE_V(kBF16, 1, 32, 0, 128, 1, 4)
  MOE_V(kBF16, 2, 32, 0, 128, 1, 4)
  MOE_V(kBF16, 1, 16, 0, 256, 1, 4)
  MOE_V(kBF16, 2, 16, 0, 256, 1, 4)
  MOE_V(kFP8, 1, 256, 0, 256, 2, 4)
  MOE_V(kFP8, 2, 256, 0, 256, 2, 4)
  MOE_V(kFP8, 1, 256, 1, 256, 2, 2)
  MOE_V(kFP8, 2, 256, 1, 256, 2, 2)
  MOE_V(kFP8, 1, 128, 0, 256, 2, 4)
  MOE_V(kFP8, 2, 128, 0, 256, 2, 4)
  MOE_V(kFP8, 1, 128, 1, 256, 2, 2)
  MOE_V(kFP8, 2, 128, 1, 128, 2, 2)
  MOE_V(kFP8, 1, 64, 0, 256, 1, 4)
  MOE_V(kFP8, 2, 64, 0, 128, 1, 4)
  MOE_V(kFP8, 1, 32, 0, 256, 2, 2)
  MOE_V(kFP8, 2, 32, 0, 128, 1, 4)
  MOE_V(kFP8, 1, 16, 0, 256, 1, 4)
  MOE_V(kFP8, 2, 16, 0, 128, 1, 4)
  MOE_V(kF32, 1, 256, 0, 128, 2, 2)
  MOE_V(kF32, 2, 256, 0, 128, 2, 2)
  MOE_V(kF32, 1, 128, 0, 128, 2, 2)
  MOE_V(kF32, 2, 128, 0, 128, 2, 2)
  MOE_V(kF32, 1, 64, 0, 128, 1, 4)
  MOE_V(kF32, 2, 64, 0, 128, 1, 4)
  MOE_V(kF32, 1, 32, 0, 128, 1, 4)
  MOE_V(kF32, 2, 32, 0, 128, 1, 4)
  MOE_V(kF32, 1, 16, 0, 128, 1, 4)
  MOE_V(kF32, 2, 16, 0, 128, 1, 4)
#undef MOE_V
  return -1;
}

template <typename F>
int dispatch(int phase, int dtype, int bm, F&& f) {
  int r = dispatch_var(phase, dtype, bm, variant_choice(), f);
  if (r == -1 && variant_choice() != 0) r = dispatch_var(phase, dtype, bm, 0, f);
  return r;
}

}  // namespace

int launch_gemm(int phase, int dtype, int bm, const GemmArgs& a, hipStream_t s) {
  return dispatch(phase, dtype, bm, [&](auto v) { return decltype(v)::launch(a, s); });
}

int gemm_tile_n(int phase, int dtype, int bm) {
  return dispatch(phase, dtype, bm, [&](auto v) { return decltype(v)::tile_n(); });
}

}  // namespace moe
