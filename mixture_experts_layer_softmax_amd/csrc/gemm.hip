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

#include <mutex>

namespace moe {

namespace {

constexpr int kRowBytes = 128;
constexpr int kThreads = 256;

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

template <int DT, int PHASE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int ES = ESize<DT>::v;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int ACH = BM * 8, BCH = BN * 8;  // 16-byte chunks per K-step
  constexpr int RA = (ACH + kThreads - 1) / kThreads;
  constexpr int RB = (BCH + kThreads - 1) / kThreads;
  static_assert(WM * WN == 4, "four waves");
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(PHASE == 2 || TN % 2 == 0, "gate/up pairs");
  static_assert(!(DT == kFP8 && PHASE == 1) || BN == 256, "FP8 h groups of 128 f");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* As = lds;                                  // [2][BM][128]
  uint8_t* Bs = lds + 2 * BM * kRowBytes;             // [2][BN][128]
  float* red = reinterpret_cast<float*>(Bs + 2 * BN * kRowBytes);  // [WN][BM]
  __shared__ int s_task;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t K = g.K, N = g.N;
  const int ksteps = static_cast<int>(K * ES / kRowBytes);
  const int kblocks = static_cast<int>(K / 128);  // FP8 scale blocks along K
  const int nblocks = static_cast<int>(N / 128);
  const int total = *g.tm.n_mtiles * g.n_tiles_n;

  for (;;) {
    if (tid == 0) s_task = atomicAdd(&g.tm.queue[g.queue_idx], 1);
    __syncthreads();
    const int task = s_task;
    if (task >= total) break;
    const int mt = task / g.n_tiles_n;
    const int nt = task - mt * g.n_tiles_n;
    const int e = g.tm.e[mt], row0 = g.tm.row0[mt], rows = g.tm.rows[mt];
    const int64_t n0 = static_cast<int64_t>(nt) * BN;

    // ---- global source of every 16-byte chunk this thread stages ----
    const uint8_t* pa[RA];
    const uint8_t* pb[RB];
#pragma unroll
    for (int j = 0; j < RA; ++j) {
      const int ci = tid + kThreads * j;
      const int r = min(ci >> 3, rows - 1);  // padding rows re-read a valid row
      const int64_t src = g.gather ? g.gather[row0 + r] : static_cast<int64_t>(row0 + r);
      pa[j] = g.A + src * g.a_row_bytes + (ci & 7) * 16;
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int ci = tid + kThreads * j;
      const int64_t n = n0 + (ci >> 3);
      int64_t col;
      const uint8_t* base;
      if (PHASE == 1) {  // combined rows: 16 gate rows, then 16 up rows, per f block
        col = (n >> 5) * 16 + (n & 15);
        base = (n & 16) ? g.B1 : g.B0;
      } else {
        col = n;
        base = g.B0;
      }
      col = min(col, N - 1);
      pb[j] = base + (static_cast<int64_t>(e) * N + col) * K * ES + (ci & 7) * 16;
    }

    uint4 ra[RA], rb[RB];
    auto gload = [&](int ks) {
      const int64_t off = static_cast<int64_t>(ks) * kRowBytes;
#pragma unroll
      for (int j = 0; j < RA; ++j)
        if (ACH % kThreads == 0 || tid + kThreads * j < ACH)
          ra[j] = *reinterpret_cast<const uint4*>(pa[j] + off);
#pragma unroll
      for (int j = 0; j < RB; ++j)
        if (BCH % kThreads == 0 || tid + kThreads * j < BCH)
          rb[j] = *reinterpret_cast<const uint4*>(pb[j] + off);
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < RA; ++j) {
        const int ci = tid + kThreads * j;
        if (ACH % kThreads == 0 || ci < ACH)
          *reinterpret_cast<uint4*>(As + buf * BM * kRowBytes + swz(ci >> 3, ci & 7)) = ra[j];
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int ci = tid + kThreads * j;
        if (BCH % kThreads == 0 || ci < BCH)
          *reinterpret_cast<uint4*>(Bs + buf * BN * kRowBytes + swz(ci >> 3, ci & 7)) = rb[j];
      }
    };

    // FP8: per token fragment i, the A-scale row of the lane's slot column
    const float* sa_row[TM];
    if constexpr (DT == kFP8) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = min(wm * WTM + 16 * i + l16, rows - 1);
        const int64_t src = g.gather ? g.gather[row0 + r] : static_cast<int64_t>(row0 + r);
        sa_row[i] = g.sa + src * kblocks;
      }
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < ksteps) gload(ks + 1);
      const uint8_t* Ab = As + cur * BM * kRowBytes;
      const uint8_t* Bb = Bs + cur * BN * kRowBytes;
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 xf[TM], wf[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i)
            xf[i] = *reinterpret_cast<const bf16x8*>(Ab + swz(wm * WTM + 16 * i + l16, kk * 4 + lg));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wf[j] = *reinterpret_cast<const bf16x8*>(Bb + swz(wn * WTN + 16 * j + l16, kk * 4 + lg));
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
        }
      } else if constexpr (DT == kF32) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          f32x4 xf[TM], wf[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i)
            xf[i] = *reinterpret_cast<const f32x4*>(Ab + swz(wm * WTM + 16 * i + l16, kk * 4 + lg));
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wf[j] = *reinterpret_cast<const f32x4*>(Bb + swz(wn * WTN + 16 * j + l16, kk * 4 + lg));
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[j][u], xf[i][u], acc[i][j], 0, 0, 0);
        }
      } else {  // FP8: one 16x16x128 MFMA per fragment pair and K block
        i32x8 xf[TM], wf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = wm * WTM + 16 * i + l16;
          i32x4 lo = *reinterpret_cast<const i32x4*>(Ab + swz(r, 2 * lg));
          i32x4 hi = *reinterpret_cast<const i32x4*>(Ab + swz(r, 2 * lg + 1));
          xf[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = wn * WTN + 16 * j + l16;
          i32x4 lo = *reinterpret_cast<const i32x4*>(Bb + swz(r, 2 * lg));
          i32x4 hi = *reinterpret_cast<const i32x4*>(Bb + swz(r, 2 * lg + 1));
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
          const float s_a = sa_row[i][ks];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf[i], z, 0, 0,
                                                                        0, 127, 0, 127);
            const float s = s_a * ((PHASE == 1 && (j & 1)) ? s_b1 : s_b0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], s, acc[i][j][r]);
          }
        }
      }
      if (ks + 1 < ksteps) lstore(cur ^ 1);
      __syncthreads();
    }

    // ---------------- epilogue ----------------
    if constexpr (PHASE == 2) {
      float* Y = reinterpret_cast<float*>(g.C);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int lr = wm * WTM + 16 * i + l16;
        if (lr >= rows) continue;
        const int64_t slot = row0 + lr;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t col = n0 + wn * WTN + 16 * j + 4 * lg;
          if (col < N) *reinterpret_cast<f32x4*>(Y + slot * N + col) = acc[i][j];
        }
      }
    } else if constexpr (DT != kFP8) {
      const int64_t fbase = ((n0 + wn * WTN) >> 1) + 4 * lg;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int lr = wm * WTM + 16 * i + l16;
        if (lr >= rows) continue;
        const int64_t slot = row0 + lr;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const int64_t col = fbase + 16 * p;
          if (col >= N) continue;
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu(acc[i][2 * p][r]) * acc[i][2 * p + 1][r];
          if constexpr (DT == kBF16) {
            uint2 v;
            v.x = f32_to_bf16_rne(h[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(h[1])) << 16);
            v.y = f32_to_bf16_rne(h[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(h[3])) << 16);
            *reinterpret_cast<uint2*>(g.C + (slot * N + col) * 2) = v;
          } else {
            *reinterpret_cast<f32x4*>(g.C + (slot * N + col) * 4) = f32x4{h[0], h[1], h[2], h[3]};
          }
        }
      }
    } else {
      // FP8 h: SwiGLU in fp32, then one scale per (slot, 128 f columns) --
      // the whole workgroup tile -- and E4M3 codes.
      float h[TM][TN / 2][4];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float m = 0.f;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            h[i][p][r] = silu(acc[i][2 * p][r]) * acc[i][2 * p + 1][r];
            m = fmaxf(m, fabsf(h[i][p][r]));
          }
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (lg == 0) red[wn * BM + wm * WTM + 16 * i + l16] = m;
      }
      __syncthreads();
      const int64_t fbase = ((n0 + wn * WTN) >> 1) + 4 * lg;
      const int fgroup = static_cast<int>(n0 / 256);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int lr = wm * WTM + 16 * i + l16;
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red[w * BM + lr]);
        if (lr >= rows) continue;
        const float s = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
        const int64_t slot = row0 + lr;
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          uint32_t packed = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) packed |= f32_to_e4m3(__fdiv_rn(h[i][p][r], s)) << (8 * r);
          *reinterpret_cast<uint32_t*>(g.C + slot * N + fbase + 16 * p) = packed;
        }
        if (wn == 0 && lg == 0) g.sc[slot * (N / 128) + fgroup] = s;
      }
    }
  }
}

template <int DT, int PHASE, int BM, int BN, int WM, int WN>
struct Variant {
  static constexpr int lds_bytes() {
    return 2 * (BM + BN) * kRowBytes + ((DT == kFP8 && PHASE == 1) ? WN * BM * 4 : 0);
  }
  static int launch(const GemmArgs& a, hipStream_t s) {
    auto kern = grouped_gemm_kernel<DT, PHASE, BM, BN, WM, WN>;
    static int grid = 0;
    static std::once_flag once;
    std::call_once(once, [&] {
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
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

// Kernel variant per (dtype, phase, tile height).
template <typename F>
int dispatch(int phase, int dtype, int bm, F&& f) {
#define MOE_V(DT, P, BM_, BN_, WM_, WN_) \
  if (dtype == DT && phase == P && bm == BM_) return f(Variant<DT, P, BM_, BN_, WM_, WN_>{});
  MOE_V(kBF16, 1, 128, 128, 2, 2)
  MOE_V(kBF16, 2, 128, 128, 2, 2)
  MOE_V(kBF16, 1, 64, 128, 1, 4)
  MOE_V(kBF16, 2, 64, 128, 1, 4)
  MOE_V(kBF16, 1, 32, 128, 1, 4)
  MOE_V(kBF16, 2, 32, 128, 1, 4)
  MOE_V(kBF16, 1, 16, 256, 1, 4)
  MOE_V(kBF16, 2, 16, 256, 1, 4)
  MOE_V(kFP8, 1, 128, 256, 2, 2)
  MOE_V(kFP8, 2, 128, 128, 2, 2)
  MOE_V(kFP8, 1, 64, 256, 1, 4)
  MOE_V(kFP8, 2, 64, 128, 1, 4)
  MOE_V(kFP8, 1, 32, 256, 2, 2)
  MOE_V(kFP8, 2, 32, 128, 1, 4)
  MOE_V(kFP8, 1, 16, 256, 1, 4)
  MOE_V(kFP8, 2, 16, 128, 1, 4)
  MOE_V(kF32, 1, 128, 128, 2, 2)
  MOE_V(kF32, 2, 128, 128, 2, 2)
  MOE_V(kF32, 1, 64, 128, 1, 4)
  MOE_V(kF32, 2, 64, 128, 1, 4)
  MOE_V(kF32, 1, 32, 128, 1, 4)
  MOE_V(kF32, 2, 32, 128, 1, 4)
  MOE_V(kF32, 1, 16, 128, 1, 4)
  MOE_V(kF32, 2, 16, 128, 1, 4)
#undef MOE_V
  return -1;
}

}  // namespace

int launch_gemm(int phase, int dtype, int bm, const GemmArgs& a, hipStream_t s) {
  return dispatch(phase, dtype, bm, [&](auto v) { return decltype(v)::launch(a, s); });
}

int gemm_tile_n(int phase, int dtype, int bm) {
  return dispatch(phase, dtype, bm, [&](auto v) { return decltype(v)::tile_n(); });
}

}  // namespace moe
