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
// Phase 2 (W2): h rows of an m-tile times the expert's down weights: Y per
// slot, fp32 on fp32 layers, bf16 on MXFP4 layers, else fp16 codes under a
// power-of-two scale per 32 columns.
//
// Scheduling: a persistent grid sized from occupancy pulls (m-tile, n-tile)
// tasks from integer atomic counters -- a work-conserving device-side tile
// queue (FlashMoE Kernel page, Architecture: the scheduler hands out work by
// readiness; MegaMoE-vs-MoE-systems page, section 2.7: a global atomic task
// counter).  Skewed experts simply own more tasks; idle CUs keep pulling.
// Padding rows exist only inside the last m-tile of an expert and are never
// stored (FlashMoE Kernel page, Communication: padding is local, just before
// compute).
//
// Operand pipeline: an NS-stage LDS ring.  Each stage holds KRB bytes of the
// contraction axis for the BM activation rows and the BN weight rows, filled
// by direct global->LDS loads (buffer_load_dwordx4 ... lds: lane L of a wave
// writes 16 bytes at the wave's LDS base + 16 L) issued NS-1 stages ahead, so
// up to (NS-1) stages of both operands are in flight per CU without passing
// through VGPRs.  Each wave waits only for its own loads of the stage it is
// about to use (vmcnt), then one barrier publishes the stage.  The source
// address of each lane is chosen so that rows land XOR-swizzled by 16-byte
// chunk, which keeps the MFMA fragment reads free of LDS bank conflicts.
//
// MFMA mapping: the weight fragment is the MFMA "A" operand and the token
// fragment the "B" operand, so the 16x16 result tile is D[n][slot]: lane l
// holds n = 4*(l/16) + r (r = 0..3) of slot l%16 -- four consecutive output
// columns of one row, which puts gate/up pairs in the same lane.
#include "device_common.hpp"
#include "launch.hpp"

#include <cstdlib>
#include <mutex>
#include <type_traits>

namespace moe {

namespace {

template <int DT>
struct ESize;
template <>
struct ESize<kF32> { static constexpr int v = 4; };
template <>
struct ESize<kBF16> { static constexpr int v = 2; };
template <>
struct ESize<kFP8> { static constexpr int v = 1; };
template <>
struct ESize<kMX4> { static constexpr int v = 1; };  // activations: MX FP8 codes

constexpr int kLdsBytes = 160 * 1024;  // LDS per CU on gfx950

// Compile-time geometry of one kernel variant.
template <int DT, int PHASE, int BM, int BN, int WM, int WN, int KRB_>
struct Geo {
  static constexpr int NW = WM * WN;
  static constexpr int kThreads = NW * 64;
  static constexpr int ES = ESize<DT>::v;
  // contraction bytes per LDS row and stage: two 16x16x32 bf16 MFMA steps,
  // four 16x16x4 fp32 steps, or one 16x16x128 FP8 step.  128-byte rows keep
  // every DMA request a whole cache line and halve the barriers per MFMA.
  // MX layers (FP4 weights): a stage spans KRB activation bytes = KRB
  // contraction elements, which the FP4 weight rows hold in KRB/2 bytes.
  static constexpr bool MX = DT == kMX4;
  static constexpr int KRB = KRB_;
  static constexpr int KRBW = MX ? KRB_ / 2 : KRB_;  // weight row bytes per stage
  static constexpr int ROWS_PER_DMA = 1024 / KRB;    // activation rows one wave-wide DMA fills
  static constexpr int ROWS_PER_DMAW = 1024 / KRBW;  // weight rows one wave-wide DMA fills
  static constexpr int ABLK = BM / ROWS_PER_DMA, BBLK = BN / ROWS_PER_DMAW;
  static constexpr int AW = (ABLK + NW - 1) / NW, BW = (BBLK + NW - 1) / NW;
  // per-stage scale DMAs (one dword per row): FP8 A-row scales; MX A-row and
  // weight-row E8M0 scale dwords (4 blocks of 32 elements each)
  static constexpr int SA_DMA = (DT == kFP8 || MX) ? (BM + 63) / 64 : 0;
  static constexpr int SB_DMA = MX ? (BN + 63) / 64 : 0;
  static constexpr int SCW = (SA_DMA + SB_DMA + NW - 1) / NW;  // scale DMAs per wave (MX)
  static constexpr int SCALE_BYTES = MX ? (SA_DMA + SB_DMA) * 256 : 0;  // per stage (MX)
  static constexpr int STAGE = BM * KRB + BN * KRBW + SCALE_BYTES;
  static constexpr int RED = (DT == kFP8 && PHASE == 1) ? WN * BM * 4 : 0;
  // FP8 activation-row scales: one 16-byte DMA per row fetches the scales
  // of four stages (a scale group) into a ring of three group buffers of
  // SA_DMA * 64 rows, after the operand ring and the row maxima
  static constexpr int SGROUP = 4;
  static constexpr int SRING_BUFS = 3;
  static constexpr int SRING = (DT == kFP8) ? SRING_BUFS * SA_DMA * 1024 : 0;
  // FP8: the tile's weight block scales for the whole contraction, two
  // columns of kWscMax floats (W1 and W3 of the tile's 128 f, or the two
  // 128-column blocks of a W2 tile), staged once per task
  static constexpr int WSC = (DT == kFP8) ? 2 * kWscMax * 4 : 0;
  static constexpr int NS0 = (kLdsBytes - RED - SRING - WSC) / STAGE;
  // small tiles (decode: HBM bound) keep more stages in flight; 16-row MX
  // tiles are small enough that two workgroups of 4 stages share a CU, which
  // streams better than one of 8 (one refills while the other starts a task)
  static constexpr int NS_CAP = BM <= 32 ? ((MX && BM == 16) ? 4 : 8) : 6;
  static constexpr int NS = NS0 > NS_CAP ? NS_CAP : NS0;
  // phase-2 output element: Y is fp32 on fp32 layers, bf16 (RNE) on MXFP4
  // layers, whose 5e-2 tolerance leaves room for that rounding, and on bf16
  // and FP8 layers fp16 codes under a power-of-two scale per 32 columns (an
  // 11-bit significand: its rounding adds at most 2^-12 of each term)
  static constexpr int YES = (DT == kF32) ? 4 : 2;
  static constexpr bool YF16 = DT == kBF16 || DT == kFP8;
  static_assert(PHASE == 1 || !YF16 || (BN / WN) % 32 == 0, "fp16 Y groups of 32 inside a wave");
  static constexpr int EPI =  // output staging, one pass per wave row
      (BM / WM) * ((PHASE == 1) ? BN / 2 : BN) * ((PHASE == 1) ? ES : YES);
  static constexpr int RING = NS * STAGE;
  static constexpr int LDS = (RING > EPI ? RING : EPI) + RED + SRING + WSC;
  static_assert(NS >= 2, "at least two LDS stages");
  // a scale group's buffer is refilled with the DMA of stage SGROUP * g,
  // issued NS - 1 stages ahead; the group that used it last (three groups
  // back) must have finished reading it by then
  static_assert(DT != kFP8 || NS - 1 < SGROUP * (SRING_BUFS - 1) + 1, "scale ring depth");
  static_assert(LDS <= kLdsBytes, "LDS budget");
  static_assert(BM % ROWS_PER_DMA == 0 && BN % ROWS_PER_DMAW == 0, "whole DMA blocks");
};

// LDS byte offset of 16-byte chunk c of row r in a tile of KRB-byte rows.
// The chunk index is XORed with bits 1.. of the row, which (measured on
// gfx950) keeps the ds_read_b128 fragment reads -- 16 consecutive rows, one
// chunk -- free of LDS bank conflicts for both 64- and 128-byte rows; keying
// on bits 0-1 or 2-3 instead halves the read rate for 64-byte rows.
template <int KRB>
__device__ __forceinline__ int swz_key(int r) {
  return (r >> 1) & (KRB / 16 - 1);
}
template <int KRB>
__device__ __forceinline__ int swz(int r, int c) {
  return r * KRB + ((c ^ swz_key<KRB>(r)) << 4);
}

// Weight tiles of the stated [K][N] layout ("k-row" tiles): a stage holds
// KS contraction rows of the tile's columns, HB bytes per row (per half:
// phase 1 keeps the tile's W1 and W3 columns in two halves).  16-byte chunk
// c of row k is stored at chunk c ^ kn_key(k), a key chosen (with a model of
// the 64 banks) so that the transposing fragment reads below -- 16 or 32
// rows at a time -- touch every bank equally often.
template <int ES, int HB>
__device__ __forceinline__ int kn_key(int k) {
  if constexpr (ES == 2) return HB >= 256 ? ((k << 2) ^ (k >> 2)) : (k ^ (k >> 1));
  else if constexpr (ES == 1) return k ^ (k >> 2) ^ (k >> 3);
  else return k;
}
template <int ES, int HB>
__device__ __forceinline__ int kn_off(int k, int byte) {
  return k * HB + ((((byte >> 4) ^ kn_key<ES, HB>(k)) & (HB / 16 - 1)) << 4) + (byte & 15);
}
typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((ext_vector_type(2))) int v2i32;
#define MOE_LDS3 __attribute__((address_space(3)))
// gfx950 transposing LDS reads.  Measured lane layout (16-lane groups, each
// lane addressing 8 bytes): the 16-bit form gives lane i element i % 4 of
// lane 4j + i / 4's 4 elements as its element j; the 8-bit form gives lane i
// byte i % 8 of lane 2j + i / 8's 8 bytes as its byte j.  So lanes that
// address 4 (or 8) consecutive columns of rows k0 + m / 4 (or k0 + m / 2)
// hand every lane 4 (or 8) consecutive rows of one column.
__device__ __forceinline__ v4i16 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS3 v4i16*)(p));
}
__device__ __forceinline__ v2i32 lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((MOE_LDS3 v2i32*)(p));
}

// s_waitcnt vmcnt(n) that leaves expcnt and lgkmcnt alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define MOE_W(N)                                                                        \
  case N:                                                                               \
    __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14)); \
    break;
  switch (n) {
    MOE_W(0) MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7)
    MOE_W(8) MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15)
    MOE_W(16) MOE_W(17) MOE_W(18) MOE_W(19) MOE_W(20) MOE_W(21) MOE_W(22) MOE_W(23)
    MOE_W(24) MOE_W(25) MOE_W(26) MOE_W(27) MOE_W(28) MOE_W(29) MOE_W(30) MOE_W(31)
    MOE_W(32) MOE_W(33) MOE_W(34) MOE_W(35) MOE_W(36) MOE_W(37) MOE_W(38) MOE_W(39)
    MOE_W(40) MOE_W(41) MOE_W(42) MOE_W(43) MOE_W(44) MOE_W(45) MOE_W(46) MOE_W(47)
    MOE_W(48) MOE_W(49) MOE_W(50) MOE_W(51) MOE_W(52) MOE_W(53) MOE_W(54) MOE_W(55)
    MOE_W(56) MOE_W(57) MOE_W(58) MOE_W(59) MOE_W(60) MOE_W(61) MOE_W(62)
    default:
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      break;
  }
#undef MOE_W
}

// wait_vmcnt with a compile-time count
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): every LDS read of this wave has returned (vmcnt
// and expcnt fields at their maxima, so they do not wait).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Direct global -> LDS loads; the LDS pointer must be wave-uniform.
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// The same 16-byte direct load through a buffer resource (base, extent):
// lane L reads voff bytes past the base (zeros past the extent) and writes
// the wave's LDS base + 16 L.  The buffer form keeps the compiler's LDS wait
// counts exact: it treats the global form as a possible LDS access of its
// own, and then makes every LDS wait behind one in flight a wait for all.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  // word 3: gfx9 raw-buffer flags (32-bit data format, no swizzle)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(min(bytes, int64_t{0x7fffffff})),
                                           0x00020000);
}
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// SiLU with the hardware exponential and reciprocal (about 2 ulp in fp32;
// h is rounded to the activation format right after).
__device__ __forceinline__ float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Workgroup barrier for the DMA ring.  __syncthreads() also emits a release
// fence whose s_waitcnt vmcnt(0) would drain every stage in flight; LDS needs
// no cache maintenance, each wave has already waited for its own loads of the
// stage (vmcnt) and for its LDS reads of the slot being refilled (their
// results fed the MFMAs), so a bare s_barrier suffices.  The empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ring_barrier that the instruction scheduler also may not move any
// instruction across (the ping-pong phases must stay whole).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

constexpr int kXcd = 8;  // XCDs (L2 domains) of the chip

// Per-XCD task queues of one grouped GEMM (see the kernel).  Task ids are
// m-tile * NT + n-tile; queue y hands out the tasks of chunks y, y+8, ...
// (chunk = GM consecutive m-tiles), n-tile-major inside a chunk.
struct TaskQueue {
  int* counters;  // [kXcd] integer pull counters, zeroed by the scan kernel
  int M, NT, GM, nchunks, xcd;
  int order;      // 0 as laid out; 1 each queue reversed; 2 each queue shuffled

  __device__ int limit(int y) const {
    const int owned = nchunks > y ? (nchunks - y + kXcd - 1) / kXcd : 0;
    return owned * GM * NT;
  }
  // task of pull number v of queue y, or -1 (the last chunk may hold fewer
  // than GM m-tiles).  A debug order first maps v through a bijection of
  // [0, limit(y)): reversal, or v -> (v * P + 12345) mod limit with P a prime
  // above any limit (so coprime to it).
  __device__ int decode(int v, int y) const {
    if (order != 0) {
      const int lim = limit(y);
      v = order == 1 ? lim - 1 - v
                     : static_cast<int>((static_cast<int64_t>(v) * 2147483629ll + 12345) % lim);
    }
    const int per_chunk = GM * NT;
    const int p = v % per_chunk;
    const int mt = (y + kXcd * (v / per_chunk)) * GM + p % GM;
    return mt < M ? mt * NT + p / GM : -1;
  }
  // pull from the own queue (s0 = 0) or start with the next XCD's (s0 = 1),
  // moving on while queues are drained; -1 once every queue is.
  __device__ int pull(int s0) const {
    for (int s = s0; s < kXcd; ++s) {
      const int y = (xcd + s) % kXcd;
      const int lim = limit(y);
      for (;;) {
        if (__hip_atomic_load(&counters[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= lim)
          break;
        const int v = atomicAdd(&counters[y], 1);
        if (v >= lim) break;
        const int t = decode(v, y);
        if (t >= 0) return t;
      }
    }
    return -1;
  }
};

// One task of the grouped GEMM: m-tile mt (rows of one expert, from the tile
// map) times column tile nt -- the K loop through the LDS ring, then the
// epilogue.  kpull() runs a few k-steps before the end (the next task's
// queue request); pre_epi() runs between the main loop and the epilogue.
// LIM (nonzero): the default loop runs the MFMAs of this wave's first LIM
// fragment rows only.
template <int DT, int PHASE, int BM, int BN, int WM, int WN, int KRB_, int SCHED, bool WKN,
          int LIM = 0, class KPull, class PreEpi>
__device__ __forceinline__ void gemm_task(const GemmArgs& g, const int mt, const int nt,
                                          const int64_t arow_base, const int64_t crow_base,
                                          KPull&& kpull,
                                          PreEpi&& pre_epi) {
  using G = Geo<DT, PHASE, BM, BN, WM, WN, KRB_>;
  constexpr int kThreads = G::kThreads, ES = G::ES, KRB = G::KRB, NS = G::NS;
  constexpr int NW = G::NW, RPD = G::ROWS_PER_DMA, RPDW = G::ROWS_PER_DMAW, KRBW = G::KRBW;
  constexpr bool MX = G::MX;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(PHASE == 2 || TN % 2 == 0, "gate/up pairs");
  static_assert(!(DT == kFP8 && PHASE == 1) || BN == 256, "FP8 h groups of 128 f");
  static_assert(!(MX && PHASE == 1) || WTN % 64 == 0, "MX h blocks of 32 f inside one wave");
  // k-row weight tiles (WKN, the stated [K][N] layout): NH halves (phase 1:
  // the tile's W1 columns, then its W3 columns) of KSW rows of HB bytes
  static_assert(!WKN || (!MX && (SCHED & 7) == 0), "k-row weight tiles: F32, BF16, FP8; default loop");
  constexpr int NH = (PHASE == 1) ? 2 : 1;
  constexpr int KSW = KRB / ES;           // contraction rows of a stage
  constexpr int HB = (BN / NH) * ES;      // bytes of one row of one half
  constexpr int HALF = KSW * HB;          // bytes of one half
  static_assert(!WKN || (HB <= 1024 && HALF % 1024 == 0 && HB % 16 == 0), "k-row DMA blocks");

  // SCHED bit 4: each wave runs the task in the instantiation for the number
  // of its fragment rows that hold a valid row (all, half or a quarter of
  // them), so the last m-tile of an expert runs no MFMAs for most of its
  // padding.  Every instantiation passes the same barriers.
  if constexpr ((SCHED & 16) && LIM == 0 && TM >= 4) {
    const int wave_row = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) / WN;
    const int valid = __builtin_amdgcn_readfirstlane(g.tm.rows[mt]) - wave_row * WTM;
    if (valid > 16 * (TM / 2))
      gemm_task<DT, PHASE, BM, BN, WM, WN, KRB_, SCHED, WKN, TM>(g, mt, nt, arow_base, crow_base,
                                                                 kpull, pre_epi);
    else if (valid > 16 * (TM / 4))
      gemm_task<DT, PHASE, BM, BN, WM, WN, KRB_, SCHED, WKN, TM / 2>(g, mt, nt, arow_base,
                                                                     crow_base, kpull, pre_epi);
    else
      gemm_task<DT, PHASE, BM, BN, WM, WN, KRB_, SCHED, WKN, TM / 4>(g, mt, nt, arow_base,
                                                                     crow_base, kpull, pre_epi);
    return;
  }
  constexpr int NR = LIM ? LIM : TM;  // fragment rows whose MFMAs run

  // LDS: NS stages of [BM rows A | BN rows B | BM A-scales (FP8)], reused by
  // the epilogue staging; then (FP8 phase 1) the per-wave row maxima.
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds + (G::RING > G::EPI ? G::RING : G::EPI));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t K = g.K, N = g.N;
  const int ksteps = static_cast<int>(K * ES / KRB);
  const int kblocks = static_cast<int>(K / 128);  // FP8 scale blocks along K
  const int nblocks = static_cast<int>(N / 128);

  const int k_pull = max(0, ksteps - 4);
  const int e = __builtin_amdgcn_readfirstlane(g.tm.e[mt]);
  const int row0 = __builtin_amdgcn_readfirstlane(g.tm.row0[mt]);
  // first row of the A operand (when not gathered) and of C: the slot row
  // row0, or arow_base / crow_base when the caller places this m-tile's rows
  // elsewhere (negative: row0)
  const int64_t arow = arow_base >= 0 ? arow_base : row0;
  const int64_t crow = crow_base >= 0 ? crow_base : row0;
  const int rows = __builtin_amdgcn_readfirstlane(g.tm.rows[mt]);
  const int64_t n0 = static_cast<int64_t>(nt) * BN;

  // ---- DMA sources of this lane: 32-bit byte offsets from wave-uniform
  // bases (the host checks that x, h and one expert's weight matrix each
  // span less than 2^31 bytes).  A wave-wide DMA fills RPD rows of KRB
  // bytes; lane L fills row L / (KRB/16), physical chunk L % (KRB/16), so it
  // loads the logical chunk that the swizzle maps there. ----
  const int64_t w_row = MX ? K / 2 : K * ES;  // weight row bytes (FP4: two per byte)
  const int64_t w_bytes = N * w_row;
  const uint8_t* b0 = g.B0 + static_cast<int64_t>(e) * w_bytes;
  const uint8_t* b1 = (PHASE == 1) ? g.B1 + static_cast<int64_t>(e) * w_bytes : b0;
  constexpr int CPRK = KRB / 16;    // 16-byte chunks per activation LDS row
  constexpr int CPRKW = KRBW / 16;  // and per weight LDS row
  const int lrow = lane / CPRK, lphys = lane % CPRK;
  const int lroww = lane / CPRKW, lphysw = lane % CPRKW;
  uint32_t oa[G::AW], ob[G::BW];
  uint32_t up_mask = 0;  // bit j: B block j of this wave comes from W3 (up)
  int my_loads = 0;      // DMA instructions this wave issues per stage
#pragma unroll
  for (int j = 0; j < G::AW; ++j) {
    const int q = wave + NW * j;
    const int r = q * RPD + lrow;
    const int logical = lphys ^ swz_key<KRB>(r);
    const int rr = min(r, rows - 1);  // padding rows re-read a valid row
    const int64_t src = g.gather ? g.gather[row0 + rr] : static_cast<int64_t>(arow + rr);
    // a block wholly past the tile's last row reads from past the end of
    // the buffer resource (offset 2^31 + k bytes), which fetches nothing
    // and returns zeros: no memory traffic for the padding rows, and the
    // same DMA count in every stage
    oa[j] = (q * RPD < rows) ? static_cast<uint32_t>(src * g.a_row_bytes + logical * 16)
                             : 0x80000000u;
    if (q < G::ABLK) ++my_loads;
  }
#pragma unroll
  for (int j = 0; j < G::BW; ++j) {
    const int q = wave + NW * j;
    if constexpr (WKN) {
      // k-row tile: block q fills 1 KB of half q / (HALF / 1024); lane L
      // fills row k, physical chunk p of it, from logical chunk p ^ key
      const int h = q / (HALF / 1024);
      const int byte = (q % (HALF / 1024)) * 1024 + 16 * lane;
      const int k = byte / HB, p = (byte % HB) / 16;
      const int logical = (p ^ kn_key<ES, HB>(k)) & (HB / 16 - 1);
      const int64_t col0 = (PHASE == 1) ? n0 / 2 : n0;
      // columns past N (the last n-tile of a ragged N) re-read the last
      // chunk of the row; they feed only columns that are never stored
      const int64_t cb = min(col0 * ES + logical * 16, N * ES - 16);
      ob[j] = static_cast<uint32_t>(k * N * ES + cb);
      if (h == 1) up_mask |= 1u << j;
      if (q < G::BBLK) ++my_loads;
      continue;
    }
    const int r = q * RPDW + lroww;
    const int logical = lphysw ^ swz_key<KRBW>(r);
    const int64_t n = n0 + r;
    int64_t col;
    if (PHASE == 1) {  // combined rows: 16 gate rows, then 16 up rows, per f block
      // the RPD rows of one DMA lie in one 16-row block (RPD divides 16 and
      // n0 is a multiple of 32), so the gate/up choice is wave-uniform
      static_assert(16 % RPDW == 0, "DMA rows inside one gate/up block");
      col = (n >> 5) * 16 + (n & 15);
      if ((q * RPDW) & 16) up_mask |= 1u << j;
    } else {
      col = n;
    }
    col = min(col, N - 1);
    ob[j] = static_cast<uint32_t>(col * w_row + logical * 16);
    if (q < G::BBLK) ++my_loads;
  }
  // FP8: this lane's A-row scale row (padded to sa_stride floats, a multiple
  // of 4, so that a scale group is one aligned 16-byte piece), and the scale
  // ring: group buffer b holds [SA_DMA * 64 rows][4 stages] floats
  uint32_t sa_off = 0;  // byte offset of that row in g.sa
  float* sring = reinterpret_cast<float*>(lds + (G::RING > G::EPI ? G::RING : G::EPI) + G::RED);
  float* wsc = sring + G::SRING / 4;  // FP8 weight block scales [2][kWscMax]
  const bool scale_dma = DT == kFP8 && wave < G::SA_DMA;
  if constexpr (DT == kFP8) {
    const int rr = min(wave * 64 + lane, rows - 1);
    const int64_t src = g.gather ? g.gather[row0 + rr] : static_cast<int64_t>(row0 + rr);
    sa_off = static_cast<uint32_t>(src * g.sa_stride * 4);
  }
  // MX: E8M0 scale dwords of this lane (4 blocks of 32 = one stage).
  // Scale DMA number c < SA_DMA covers activation rows 64c.. ([rows][K/32]
  // bytes: the next stage's dword follows), the others weight rows
  // 64(c - SA_DMA).. of the tile (packed [E][K/128][N] dwords: a stage's
  // dwords of consecutive rows are contiguous, the next stage is N dwords
  // on); wave w issues c = w, w + NW, ...
  const uint8_t* msc[G::SCW > 0 ? G::SCW : 1];
  uint32_t mstep[G::SCW > 0 ? G::SCW : 1];
  if constexpr (MX) {
    const int64_t kb32 = K / 32;
#pragma unroll
    for (int u = 0; u < G::SCW; ++u) {
      const int c = wave + NW * u;
      msc[u] = nullptr;
      mstep[u] = 4;
      if (c < G::SA_DMA) {
        const int rr = min(c * 64 + lane, rows - 1);
        const int64_t src = g.gather ? g.gather[row0 + rr] : static_cast<int64_t>(row0 + rr);
        msc[u] = reinterpret_cast<const uint8_t*>(g.sa) + src * kb32;
        ++my_loads;
      } else if (c < G::SA_DMA + G::SB_DMA) {
        const int64_t n = n0 + (c - G::SA_DMA) * 64 + lane;
        int64_t col = (PHASE == 1) ? (n >> 5) * 16 + (n & 15) : n;
        col = min(col, N - 1);
        const float* sb = (PHASE == 1 && (n & 16)) ? g.sb1 : g.sb0;
        msc[u] = reinterpret_cast<const uint8_t*>(sb) + (static_cast<int64_t>(e) * N * kb32 + col * 4);
        mstep[u] = static_cast<uint32_t>(N * 4);
        ++my_loads;
      }
    }
  }

  // buffer resources of the activation rows, this expert's weight rows and
  // (FP8) the activation-row scales
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb0 = buffer_rsrc(b0, w_bytes), rb1 = buffer_rsrc(b1, w_bytes);
  const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(g.sa, DT == kFP8 ? g.sa_bytes : 0);
  auto dma_a = [&](uint32_t off, void* dst) { dma16b(ra, off, dst); };
  auto dma_b = [&](bool up, uint32_t off, void* dst) { dma16b(up ? rb1 : rb0, off, dst); };
  // weight bytes between consecutive stages: KRBW along a packed row, or KSW
  // rows of the stated layout
  const uint32_t w_kstride = WKN ? static_cast<uint32_t>(KSW * N * ES) : KRBW;
  // k-row tiles: LDS byte offset of the 4 (16-bit) / 8 (8-bit) bytes this
  // lane addresses for the transposing read of rows k0 + .. of tile column
  // block cb (16 columns, in the phase-1 combined order)
  auto kn_addr = [&](int cb_col, int k, int colbyte) {  // (from the stage base)
    const int blk = cb_col / 16;
    const int h = (PHASE == 1) ? (blk & 1) : 0;
    const int c0 = (PHASE == 1) ? (blk >> 1) * 16 : cb_col;
    return BM * KRB + h * HALF + kn_off<ES, HB>(k, c0 * ES + colbyte);
  };

// DMA of stage KS: the activation rows (and FP8 row scales) when DO_A, the
// weight rows when DO_B
#define MOE_ISSUE_PART(KS, DO_A, DO_B)                                                   \
do {                                                                                   \
  uint8_t* st_ = lds + ((KS) % NS) * G::STAGE;                                         \
  const uint32_t ko_ = static_cast<uint32_t>(KS) * KRB;                                \
  if (DO_A) {                                                                          \
    _Pragma("unroll") for (int j = 0; j < G::AW; ++j) {                                \
      const int q = wave + NW * j;                                                     \
      if (G::ABLK % NW == 0 || q < G::ABLK) dma_a(oa[j] + ko_, st_ + q * 1024);          \
    }                                                                                  \
    if (DT == kFP8 && scale_dma && (KS) % G::SGROUP == 0)                              \
      dma16b(rsa, sa_off + (KS) * 4,                                                   \
             sring + ((KS) / G::SGROUP) % G::SRING_BUFS * (G::SA_DMA * 256) + wave * 256);  \
  }                                                                                    \
  if (DO_B) {                                                                          \
    const uint32_t kw_ = static_cast<uint32_t>(KS) * w_kstride;                        \
    _Pragma("unroll") for (int j = 0; j < G::BW; ++j) {                                \
      const int q = wave + NW * j;                                                     \
      if (G::BBLK % NW == 0 || q < G::BBLK)                                            \
        dma_b((up_mask >> j) & 1u, ob[j] + kw_, st_ + BM * KRB + q * 1024);              \
    }                                                                                  \
    if (MX) {                                                                          \
      _Pragma("unroll") for (int u = 0; u < G::SCW; ++u) {                             \
        const int c = wave + NW * u;                                                   \
        if (c < G::SA_DMA + G::SB_DMA)                                                 \
          dma4(msc[u] + (KS) * mstep[u], st_ + BM * KRB + BN * KRBW + c * 256);        \
      }                                                                                \
    }                                                                                  \
  }                                                                                    \
} while (0)
#define MOE_ISSUE(KS) MOE_ISSUE_PART(KS, true, true)

  // FP8: the weight block scales of this tile are read once per task, by
  // the whole workgroup, into two LDS columns: W1 and W3 of block n0 / 256
  // (phase 1), or blocks n0 / 128 and n0 / 128 + 1 (phase 2; a block past
  // the last is clamped to it, and feeds only columns that are never
  // stored).  Each k-step then reads its scale from LDS: no scalar loads
  // (which would make every LDS wait in the loop a wait for all) and no
  // vector loads among the DMAs.  Wave wn reads column wsc_col.
  constexpr int WSCU = (2 * kWscMax + kThreads - 1) / kThreads;  // entries per thread
  float wsc_v[WSCU];
  int wsc_col = 0;
  if constexpr (DT == kFP8) {
    wsc_col = (PHASE == 1) ? 0 : (wn * WTN) / 128;
#pragma unroll
    for (int u = 0; u < WSCU; ++u) {
      wsc_v[u] = 0.f;
      const int idx = tid + kThreads * u;  // column idx / kWscMax, block idx % kWscMax
      const int c = idx / kWscMax, kb = idx % kWscMax;
      if (c < 2 && kb < kblocks) {
        const int nb = (PHASE == 1) ? static_cast<int>(n0 / 256)
                                    : min(nblocks - 1, static_cast<int>(n0 / 128) + c);
        const float* src = (PHASE == 1 && c == 1) ? g.sb1 : g.sb0;
        wsc_v[u] = src[(static_cast<int64_t>(e) * kblocks + kb) * nblocks + nb];
      }
    }
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < ksteps) MOE_ISSUE(p);
  if constexpr (DT == kFP8) {
    // (the previous task's reads of these columns ended before its epilogue
    // barrier; the first stage barrier below publishes the new ones)
#pragma unroll
    for (int u = 0; u < WSCU; ++u)
      if (tid + kThreads * u < 2 * kWscMax) wsc[tid + kThreads * u] = wsc_v[u];
    wait_lgkmcnt0();
  }

  constexpr int LOOP = SCHED & 7;  // main-loop schedule; bit 3: h / fp16 Y stored from registers
  if constexpr (LOOP == 4) {
    // Two MFMA k-steps per stage (128-byte rows, two stages), the second
    // k-step's fragments read while the first one's MFMAs run: row by row
    // into a second weight-fragment set and into the activation fragment
    // the row's MFMAs have just consumed.  Only the first k-step's reads
    // after each stage barrier are exposed.  The next stage's DMA goes out
    // one instruction per MFMA row of the first k-step.
    static_assert(DT == kBF16 && KRB == 128 && NS == 2, "bf16, 128-byte rows, two stages");
    static_assert(G::ABLK % NW == 0 && G::BBLK % NW == 0, "every wave issues AW + BW DMAs");
    static_assert(G::AW + G::BW <= TM, "one DMA per MFMA row");
    // fragment j / i of a k-step: base + 16 rows further (the swizzle key of
    // row r + 16 equals that of row r)
    const int rw0 = BM * KRB + swz<KRB>(wn * WTN + l16, lg);
    const int rw1 = BM * KRB + swz<KRB>(wn * WTN + l16, 4 + lg);
    const int rx0 = swz<KRB>(wm * WTM + l16, lg);
    const int rx1 = swz<KRB>(wm * WTM + l16, 4 + lg);
    auto main_loop = [&](auto compute_c) {
      constexpr bool kCompute = decltype(compute_c)::value;
      bf16x8 xf[TM], wa[TN], wb[TN];
      for (int ks = 0; ks < ksteps; ++ks) {
        wait_vmcnt_c<0>();  // own loads of stage ks (the only stage in flight)
        ring_barrier();     // everyone's; and stage ks - 1's slot is free
        if (ks == k_pull) kpull();
        const bool refill = ks + 1 < ksteps;
        const uint8_t* St = lds + (ks & 1) * G::STAGE;
        uint8_t* st_n = lds + ((ks + 1) & 1) * G::STAGE;
        const uint32_t ko_n = static_cast<uint32_t>(ks + 1) * KRB;
        if constexpr (kCompute) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wa[j] = *reinterpret_cast<const bf16x8*>(St + rw0 + 16 * j * KRB);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            xf[i] = *reinterpret_cast<const bf16x8*>(St + rx0 + 16 * i * KRB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (kCompute) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[j], xf[i], acc[i][j], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (refill) {
            if (i < G::AW) {
              dma16b(ra, oa[i] + ko_n, st_n + (wave + NW * i) * 1024);
            } else if (i < G::AW + G::BW) {
              const int u = i - G::AW;
              dma16b((up_mask >> u) & 1u ? rb1 : rb0, ob[u] + ko_n,
                     st_n + BM * KRB + (wave + NW * u) * 1024);
            }
          }
          if constexpr (kCompute) {
            if (i < TN) wb[i] = *reinterpret_cast<const bf16x8*>(St + rw1 + 16 * i * KRB);
            xf[i] = *reinterpret_cast<const bf16x8*>(St + rx1 + 16 * i * KRB);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kCompute) {
#pragma unroll
          for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[j], xf[i], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    if (wm * WTM < rows)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  } else if constexpr (LOOP == 2) {
    // Interleaved DMA: each k-step of a stage reads its fragments, then runs
    // its MFMAs with one DMA instruction of the next stage between every
    // few of them (the activation rows' DMAs with the first k-step, the
    // weight rows' with the second).  Issued as one block, a wave's DMA
    // instructions stall its in-order issue until the memory pipeline
    // accepts them, which delays its MFMAs; spread out, they drain behind
    // the MFMAs.  Measured in isolation on a 256 x 256 stage fed from L2:
    // 3022 instead of 3437 clocks per stage (the MFMAs alone: 2075).
    static_assert(DT == kBF16 && KRB == 128, "interleaved DMA: bf16, two k-steps per stage");
    constexpr int MA = (TM * TN + G::AW - 1) / G::AW;  // MFMAs after each activation DMA
    constexpr int MB = (TM * TN + G::BW - 1) / G::BW;  // and after each weight DMA
    const bool compute = wm * WTM < rows;
    for (int ks = 0; ks < ksteps; ++ks) {
      const int ahead = min(NS - 2, ksteps - 1 - ks);
      wait_vmcnt(ahead * my_loads);
      ring_barrier();
      if (ks == k_pull) kpull();
      const bool refill = ks + NS - 1 < ksteps;
      const int kn = ks + NS - 1;
      uint8_t* st_n = lds + (kn % NS) * G::STAGE;
      const uint32_t ko_n = static_cast<uint32_t>(kn) * KRB;
      const uint8_t* Ab = lds + (ks % NS) * G::STAGE;
      const uint8_t* Bb = Ab + BM * KRB;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 wf[TN], xf[TM];
        if (compute) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wf[j] = *reinterpret_cast<const bf16x8*>(
                Bb + swz<KRB>(wn * WTN + 16 * j + l16, kk * 4 + lg));
#pragma unroll
          for (int i = 0; i < TM; ++i)
            xf[i] = *reinterpret_cast<const bf16x8*>(
                Ab + swz<KRB>(wm * WTM + 16 * i + l16, kk * 4 + lg));
        }
        constexpr int ND = 4;  // DMA slots of this k-step (A: AW, B: BW, at most 4 each)
        static_assert(G::AW <= ND && G::BW <= ND, "DMA slots per k-step");
        const int MPD = (kk == 0) ? MA : MB;  // (kk is unrolled: a constant)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < ND; ++u) {
          if (kk == 0) {
            const int q = wave + NW * u;
            if (refill && u < G::AW && (G::ABLK % NW == 0 || q < G::ABLK))
              dma_a(oa[u] + ko_n, st_n + q * 1024);
          } else {
            const int q = wave + NW * u;
            if (refill && u < G::BW && (G::BBLK % NW == 0 || q < G::BBLK))
              dma_b((up_mask >> u) & 1u, ob[u] + static_cast<uint32_t>(kn) * KRBW,
                    st_n + BM * KRB + q * 1024);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (compute) {
#pragma unroll
            for (int m = u * MPD; m < (u + 1) * MPD && m < TM * TN; ++m) {
              const int i = m / TN, j = m % TN;
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else if constexpr (LOOP == 1) {
    // Ping-pong schedule: the two waves of each SIMD (wave row wm = 0 and
    // wm = 1) run half a stage apart.  While one runs the stage's 64 MFMAs
    // from registers at raised priority, the other reads its fragments of
    // the next stage from LDS and issues its share of the DMA, so the matrix
    // core of every SIMD always has one wave with a dense MFMA cluster; the
    // barrier between two phases is where the waves trade roles.  Group 1
    // starts one barrier late and group 0 finishes one barrier late, so
    // both pass the same number of barriers.
    //   barrier 2s:   stage s is in LDS (both groups waited for their own
    //                 loads of it); group 0 reads it, group 1 runs stage s-1
    //   barrier 2s+1: group 0 runs stage s, group 1 reads it
    // Stage s+1 goes into the slot of stage s-1, which both groups finished
    // reading by barrier 2s; each group issues its share of it in the phase
    // after barrier 2s (group 0 before its reads, group 1 before its
    // MFMAs) and waits for it before barrier 2s+2.
    static_assert(DT == kBF16 && NS == 2 && WM == 2 && KRB == 128,
                  "ping-pong: bf16, two stages, two wave rows");
    const bool late = wm == 1;
    const bool compute = wm * WTM < rows;
    wait_vmcnt(0);
    phase_barrier();  // stage 0 is in LDS
    if (late) {
      if (1 < ksteps) MOE_ISSUE(1);
      phase_barrier();
    }
    bf16x8 xf[2][TM], wf[2][TN];
    for (int ks = 0; ks < ksteps; ++ks) {
      const uint8_t* Ab = lds + (ks & 1) * G::STAGE;
      const uint8_t* Bb = Ab + BM * KRB;
      // ---- load phase: this wave's fragments of stage ks ----
      if (!late && ks + 1 < ksteps) MOE_ISSUE(ks + 1);
      if (ks == k_pull) kpull();
      if (compute) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            wf[kk][j] = *reinterpret_cast<const bf16x8*>(
                Bb + swz<KRB>(wn * WTN + 16 * j + l16, kk * 4 + lg));
#pragma unroll
          for (int i = 0; i < TM; ++i)
            xf[kk][i] = *reinterpret_cast<const bf16x8*>(
                Ab + swz<KRB>(wm * WTM + 16 * i + l16, kk * 4 + lg));
        }
      }
      if (late) wait_vmcnt(0);  // own share of stage ks + 1 has landed
      wait_lgkmcnt0();          // fragments in registers before the slot is refilled
      phase_barrier();
      // ---- compute phase: the 64 MFMAs of stage ks ----
      if (late && ks + 2 < ksteps) MOE_ISSUE(ks + 2);
      if (compute) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[kk][j], xf[kk][i], acc[i][j],
                                                                   0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
      }
      if (!late) wait_vmcnt(0);  // own share of stage ks + 1 has landed
      phase_barrier();
    }
    if (!late) phase_barrier();
  } else
  for (int ks = 0; ks < ksteps; ++ks) {
    // my loads of stage ks have landed once at most `ahead` later stages
    // are still in flight; the barrier then publishes everyone's loads and
    // guarantees every wave is done with the slot reloaded below
    const int ahead = min(NS - 2, ksteps - 1 - ks);
    // (FP8: a scale-group DMA rides with the stages whose index is a
    // multiple of SGROUP; count those among the stages still in flight)
    const int groups_ahead =
        (DT == kFP8 && scale_dma && ahead > 0)
            ? (ks + ahead) / G::SGROUP - ks / G::SGROUP
            : 0;
    wait_vmcnt(ahead * my_loads + groups_ahead);
    ring_barrier();
    if (ks == k_pull) kpull();
    // bf16 stages hold two MFMA k-steps: the weight rows of the next stage
    // are requested after the first one, which spreads the DMA's LDS writes
    // over the stage instead of piling them onto its first fragment reads
    constexpr bool kSplitDma = (DT == kBF16) && (KRB / 64 == 2);
    const bool refill = ks + NS - 1 < ksteps;
    if (refill) MOE_ISSUE_PART(ks + NS - 1, true, !kSplitDma);
    float sb_cur0 = 0.f, sb_cur1 = 0.f;  // FP8 weight block scales of this k-step
    if constexpr (DT == kFP8) {
      sb_cur0 = wsc[wsc_col * kWscMax + ks];
      if (PHASE == 1) sb_cur1 = wsc[kWscMax + ks];
    }
    const uint8_t* Ab = lds + (ks % NS) * G::STAGE;
    const uint8_t* Bb = Ab + BM * KRB;
    const uint8_t* Sb = Bb + BN * KRBW;  // per-stage scale dwords
    // A wave whose rows are all padding skips the step; a partly valid
    // wave computes its padding rows too (their results are never stored),
    // which keeps the fragment loop free of branches.
    const bool compute = wm * WTM < rows;
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int kk = 0; kk < KRB / 64; ++kk) {
        if (kSplitDma && kk == 1 && refill) MOE_ISSUE_PART(ks + NS - 1, false, true);
        if (!compute) continue;
        bf16x8 wf[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (WKN) {
            // rows 32 kk + 8 lg + 0..7 of column wn WTN + 16 j + l16
            const int k0 = kk * 32 + 8 * lg + (l16 >> 2);
            const v4i16 lo = lds_tr16(Ab + kn_addr(wn * WTN + 16 * j, k0, 8 * (l16 & 3)));
            const v4i16 hi = lds_tr16(Ab + kn_addr(wn * WTN + 16 * j, k0 + 4, 8 * (l16 & 3)));
            typedef __attribute__((ext_vector_type(8))) short v8i16;
            wf[j] = __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1],
                                                     hi[2], hi[3]});
          } else {
            wf[j] = *reinterpret_cast<const bf16x8*>(
                Bb + swz<KRB>(wn * WTN + 16 * j + l16, kk * 4 + lg));
          }
        }
        // every fragment read of the step is issued before the MFMAs (LDS
        // latency then overlaps the MFMAs instead of stalling each pair of
        // fragments)
        bf16x8 xf[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i)
          xf[i] = *reinterpret_cast<const bf16x8*>(Ab + swz<KRB>(wm * WTM + 16 * i + l16, kk * 4 + lg));
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NR + TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NR * TN, 0);
      }
    } else if constexpr (DT == kF32) {
      if (!compute) continue;
      f32x4 wf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (WKN) {  // rows 4 lg + u of column wn WTN + 16 j + l16
#pragma unroll
          for (int u = 0; u < 4; ++u)
            wf[j][u] = *reinterpret_cast<const float*>(
                Ab + kn_addr(wn * WTN + 16 * j, 4 * lg + u, 4 * l16));
        } else {
          wf[j] = *reinterpret_cast<const f32x4*>(Bb + swz<KRB>(wn * WTN + 16 * j + l16, lg));
        }
      }
#define MOE_F32_ROWS(SKIP)                                                                \
_Pragma("unroll") for (int i = 0; i < TM; ++i) {                                        \
  if (SKIP) break;                                                                      \
  const f32x4 xf =                                                                      \
      *reinterpret_cast<const f32x4*>(Ab + swz<KRB>(wm * WTM + 16 * i + l16, lg));      \
  _Pragma("unroll") for (int u = 0; u < 4; ++u)                                         \
  _Pragma("unroll") for (int j = 0; j < TN; ++j)                                        \
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[j][u], xf[u], acc[i][j], 0, 0, 0); \
}
      MOE_F32_ROWS(false)
#undef MOE_F32_ROWS
    } else if constexpr (MX) {
      // FP4 weights x MX FP8 activations: one scaled 16x16x128 MFMA per
      // fragment pair; the E8M0 block scales are MFMA operands.  Measured
      // operand layout: FP4 lane group lg holds 32 elements in its 16 bytes
      // (low nibble first) and, in both operands, lane group lg's scale
      // byte governs exactly those 32 elements; FP8 lane group lg pairs its
      // bytes 0-15 and 16-31 with half (lg & 1) of FP4 groups lg >> 1 and
      // (lg >> 1) + 2.  So contraction block lg (32 elements) of the step
      // goes to FP4 lane group lg in order, the FP8 lanes take 16-byte
      // chunks lg and lg + 4 of the activation row, and each lane passes
      // its own row's scale byte of block lg.
      if (!compute) continue;
      const uint32_t* sa_st = reinterpret_cast<const uint32_t*>(Sb);
      const uint32_t* sw_st = sa_st + G::SA_DMA * 64;
      i32x8 wf[TN];
      int wsc[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WTN + 16 * j + l16;
        const i32x4 c = *reinterpret_cast<const i32x4*>(Bb + swz<KRBW>(r, lg));
        wf[j] = i32x8{c[0], c[1], c[2], c[3], 0, 0, 0, 0};
        wsc[j] = static_cast<int>((sw_st[r] >> (8 * lg)) & 0xffu);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + 16 * i + l16;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(Ab + swz<KRB>(r, lg));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(Ab + swz<KRB>(r, lg + 4));
        const i32x8 xf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const int xsc = static_cast<int>((sa_st[r] >> (8 * lg)) & 0xffu);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf, acc[i][j], 4, 0,
                                                                       0, wsc[j], 0, xsc);
      }
    } else {  // FP8: one 16x16x128 MFMA per fragment pair and 128-K block
      if (!compute) continue;
      i32x8 wf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (WKN) {
          // rows 32 lg + 0..31 of column wn WTN + 16 j + l16, 8 per read
          v2i32 t[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            t[rr] = lds_tr8(Ab + kn_addr(wn * WTN + 16 * j, 32 * lg + 8 * rr + (l16 >> 1),
                                         8 * (l16 & 1)));
          wf[j] = i32x8{t[0][0], t[0][1], t[1][0], t[1][1], t[2][0], t[2][1], t[3][0], t[3][1]};
        } else {
          const int r = wn * WTN + 16 * j + l16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(Bb + swz<KRB>(r, 2 * lg));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(Bb + swz<KRB>(r, 2 * lg + 1));
          wf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      // this stage's column of the scale group buffer: [row][4 stages]
      const float* sa_st = sring + (ks / G::SGROUP) % G::SRING_BUFS * (G::SA_DMA * 256) +
                           ks % G::SGROUP;
      const float s_b0 = sb_cur0, s_b1 = sb_cur1;
      // Software pipeline over the NR fragment rows: row i + 1's activation
      // fragment and row scale are read from LDS while row i's TN block
      // products run on the MFMA, and row i - 1's products are scaled
      // (s_x * s_w, fp32) into the accumulators behind them, so neither the
      // LDS latency nor the MFMA result latency stalls the wave.
      i32x8 xf[2];
      float sa[2];
      auto load_row = [&](int i, i32x8& x, float& s_x) {
        const int r = wm * WTM + 16 * i + l16;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(Ab + swz<KRB>(r, 2 * lg));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(Ab + swz<KRB>(r, 2 * lg + 1));
        x = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        s_x = sa_st[4 * r];
      };
      load_row(0, xf[0], sa[0]);
      f32x4 pp[TN];
      float spg = 0.f, spu = 0.f;
#pragma unroll
      for (int i = 0; i <= NR; ++i) {
        f32x4 pc[TN];
        float scg = 0.f, scu = 0.f;
        if (i + 1 < NR) load_row(i + 1, xf[(i + 1) & 1], sa[(i + 1) & 1]);
        if (i < NR) {
          scg = sa[i & 1] * s_b0;
          scu = sa[i & 1] * s_b1;
#pragma unroll
          for (int j = 0; j < TN; ++j)
            pc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                wf[j], xf[i & 1], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        }
        if (i > 0) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const float sc = (PHASE == 1 && (j & 1)) ? spu : spg;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i - 1][j][q] = __builtin_fmaf(pp[j][q], sc, acc[i - 1][j][q]);
          }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) pp[j] = pc[j];
        spg = scg;
        spu = scu;
      }
    }
  }
#undef MOE_ISSUE
#undef MOE_ISSUE_PART

  pre_epi();

  // ---------------- epilogue ----------------
  // Output rows are staged in LDS (free after the main loop's last
  // barrier) so that every global store is a 16-byte piece of a contiguous
  // row segment: the whole tile in one pass when it fits in the ring, else
  // one pass per wave row.  Staged rows are XOR-swizzled by 16-byte chunk to
  // keep the fragment writes off a single bank group.
  {
    constexpr int OUT_COLS = (PHASE == 1) ? BN / 2 : BN;
    constexpr int OUT_ES = (PHASE == 1) ? ES : G::YES;
    constexpr int ROWB = OUT_COLS * OUT_ES;
    constexpr int CPR = ROWB / 16;
    constexpr int XM = (CPR >= 16 ? 16 : CPR) - 1;
    constexpr int PASSES = (BM * ROWB <= G::RING - 16) ? 1 : WM;
    constexpr int PROWS = BM / PASSES;  // rows per pass
    static_assert(PROWS * ROWB <= (G::RING > G::EPI ? G::RING : G::EPI), "staging fits");
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
    }
    // SCHED bit 3, phase 1 (bf16 or FP8 h): h stored straight from the
    // accumulators -- a lane holds four consecutive h columns of one row, so
    // one store writes 16 rows x 32 (bf16) or 16 (FP8) bytes; FP8 first
    // gathers the row maxima of all waves through LDS (one barrier)
    if constexpr ((SCHED & 8) && PHASE == 1 && (DT == kBF16 || DT == kFP8)) {
      if constexpr (DT == kFP8) __syncthreads();  // the row maxima are in
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (wm * WTM + 16 * i >= rows) break;  // padding rows are not stored
        const int lr = wm * WTM + 16 * i + l16;
        if (lr >= rows) continue;
        float rsc = 1.0f;
        if constexpr (DT == kFP8) {
          float amax = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red[w * BM + lr]);
          const float sc = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
          rsc = __fdiv_rn(1.0f, sc);
          if (wn == 0 && lg == 0) g.sc[static_cast<int64_t>(row0 + lr) * g.sc_stride + n0 / 256] = sc;
        }
#pragma unroll
        for (int p = 0; p < TN / 2; ++p) {
          const int64_t col = col0 + wn * (WTN / 2) + 16 * p + 4 * lg;
          if (col >= N) continue;
          uint8_t* dst = g.C + (static_cast<int64_t>(crow + lr) * N + col) * ES;
          if constexpr (DT == kFP8) {
            *reinterpret_cast<uint32_t*>(dst) =
                f32x4_to_e4m3x4(acc[i][2 * p][0] * rsc, acc[i][2 * p][1] * rsc,
                                acc[i][2 * p][2] * rsc, acc[i][2 * p][3] * rsc);
          } else {
            float h[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              h[q4] = silu(acc[i][2 * p][q4]) * acc[i][2 * p + 1][q4];
            u32x2 v;
            v.x = f32x2_to_bf16x2_rne(h[0], h[1]);
            v.y = f32x2_to_bf16x2_rne(h[2], h[3]);
            *reinterpret_cast<u32x2*>(dst) = v;
          }
        }
      }
      return;
    }
    // SCHED bit 3, fp16 Y: stored straight from the accumulators, without
    // staging or barriers -- each lane holds four consecutive columns (8
    // bytes) of one row, so one store writes 16 rows x 32 bytes
    if constexpr ((SCHED & 8) && PHASE == 2 && G::YF16) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (wm * WTM + 16 * i >= rows) break;  // padding rows are not stored
        const int lr = wm * WTM + 16 * i + l16;
#pragma unroll
        for (int gq = 0; gq < TN / 2; ++gq) {
          float m = 0.f;
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) m = fmaxf(m, fabsf(acc[i][2 * gq + pp][q4]));
          m = fmaxf(m, __shfl_xor(m, 16, 64));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          const int x = fp16_group_exponent(m);
          const float rs = exp2_int(-x);
          const int64_t gcol = col0 + wn * WTN + 32 * gq;
          if (lr < rows && gcol < N) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int j = 2 * gq + pp;
              u32x2 v;
              v.x = f32x2_to_f16x2_rne(acc[i][j][0] * rs, acc[i][j][1] * rs);
              v.y = f32x2_to_f16x2_rne(acc[i][j][2] * rs, acc[i][j][3] * rs);
              u32x2* dst = reinterpret_cast<u32x2*>(
                  g.C + (static_cast<int64_t>(crow + lr) * N + gcol + 16 * pp + 4 * lg) * 2);
              if (g.stream_c)
                __builtin_nontemporal_store(v, dst);
              else
                *dst = v;
            }
            if (lg == 0)
              g.ce[static_cast<int64_t>(crow + lr) * (N / 32) + gcol / 32] =
                  static_cast<uint8_t>(x + 127);
          }
        }
      }
      return;
    }
    __syncthreads();  // every wave is done with the ring (and the row maxima are in)

    for (int pass = 0; pass < PASSES; ++pass) {
      if ((wm * WTM) / PROWS == pass) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int lr = wm * WTM + 16 * i + l16;  // row within the tile
          const int r = lr - pass * PROWS;          // row within this pass
          if constexpr (PHASE == 2 && G::YES == 4) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
              *reinterpret_cast<f32x4*>(stage + st_off(r, (wn * WTN + 16 * j + 4 * lg) * 4)) =
                  acc[i][j];
          } else if constexpr (PHASE == 2 && MX) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              u32x2 v;
              v.x = f32x2_to_bf16x2_rne(acc[i][j][0], acc[i][j][1]);
              v.y = f32x2_to_bf16x2_rne(acc[i][j][2], acc[i][j][3]);
              *reinterpret_cast<u32x2*>(stage + st_off(r, (wn * WTN + 16 * j + 4 * lg) * 2)) = v;
            }
          } else if constexpr (PHASE == 2) {
            // fp16 Y under a power-of-two scale per 32 columns of the row
            // (two 16-column fragments, held by the four lanes of this row):
            // the group amax sets the exponent, then fp16 codes of Y * 2^-x
#pragma unroll
            for (int gq = 0; gq < TN / 2; ++gq) {
              float m = 0.f;
#pragma unroll
              for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) m = fmaxf(m, fabsf(acc[i][2 * gq + pp][q4]));
              m = fmaxf(m, __shfl_xor(m, 16, 64));
              m = fmaxf(m, __shfl_xor(m, 32, 64));
              const int x = fp16_group_exponent(m);
              const float rs = exp2_int(-x);
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const int j = 2 * gq + pp;
                u32x2 v;
                v.x = f32x2_to_f16x2_rne(acc[i][j][0] * rs, acc[i][j][1] * rs);
                v.y = f32x2_to_f16x2_rne(acc[i][j][2] * rs, acc[i][j][3] * rs);
                *reinterpret_cast<u32x2*>(stage + st_off(r, (wn * WTN + 16 * j + 4 * lg) * 2)) = v;
              }
              // (one byte per row and group, straight from the lanes: staging
              // them through LDS measured slower on the FP8 layer)
              const int64_t gcol = col0 + wn * WTN + 32 * gq;
              if (lg == 0 && lr < rows && gcol < N)
                g.ce[static_cast<int64_t>(crow + lr) * (N / 32) + gcol / 32] =
                    static_cast<uint8_t>(x + 127);
            }
          } else if constexpr (MX) {
            // h = SiLU(gate) * up; each block of 32 h columns (two 16-column
            // fragments, held by the four lanes of this row) gets its MX FP8
            // exponent from the block amax, then E4M3 codes of h * 2^-X
#pragma unroll
            for (int qb = 0; qb < TN / 4; ++qb) {
              float h[2][4];
              float m = 0.f;
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const int p = 2 * qb + pp;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                  h[pp][q4] = silu(acc[i][2 * p][q4]) * acc[i][2 * p + 1][q4];
                  m = fmaxf(m, fabsf(h[pp][q4]));
                }
              }
              m = fmaxf(m, __shfl_xor(m, 16, 64));
              m = fmaxf(m, __shfl_xor(m, 32, 64));
              const int x = mx_exponent_e4m3(m);
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const uint32_t packed = f32x4_to_e4m3x4(
                    __builtin_ldexpf(h[pp][0], -x), __builtin_ldexpf(h[pp][1], -x),
                    __builtin_ldexpf(h[pp][2], -x), __builtin_ldexpf(h[pp][3], -x));
                *reinterpret_cast<uint32_t*>(
                    stage + st_off(r, wn * (WTN / 2) + 16 * (2 * qb + pp) + 4 * lg)) = packed;
              }
              if (lg == 0 && lr < rows)
                reinterpret_cast<uint8_t*>(g.sc)[static_cast<int64_t>(row0 + lr) * (N / 32) +
                                                 (col0 + wn * (WTN / 2) + 32 * qb) / 32] =
                    static_cast<uint8_t>(x + 127);
            }
          } else if constexpr (DT == kFP8) {
            float amax = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red[w * BM + lr]);
            const float sc = (amax == 0.f) ? 1.0f : __fdiv_rn(amax, 448.0f);
            // h / sc as h times the row's rounded reciprocal: within a few
            // fp32 ulp of the quotient, far inside the slack the stored h
            // is held to, for one division per row instead of per element
            const float rsc = __fdiv_rn(1.0f, sc);
#pragma unroll
            for (int p = 0; p < TN / 2; ++p) {
              const uint32_t packed =
                  f32x4_to_e4m3x4(acc[i][2 * p][0] * rsc, acc[i][2 * p][1] * rsc,
                                  acc[i][2 * p][2] * rsc, acc[i][2 * p][3] * rsc);
              *reinterpret_cast<uint32_t*>(stage + st_off(r, wn * (WTN / 2) + 16 * p + 4 * lg)) =
                  packed;
            }
            if (wn == 0 && lg == 0 && lr < rows)
              g.sc[static_cast<int64_t>(row0 + lr) * g.sc_stride + n0 / 256] = sc;
          } else {
#pragma unroll
            for (int p = 0; p < TN / 2; ++p) {
              float h[4];
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                h[q4] = silu(acc[i][2 * p][q4]) * acc[i][2 * p + 1][q4];
              const int cb = (wn * (WTN / 2) + 16 * p + 4 * lg) * ES;
              if constexpr (DT == kBF16) {
                u32x2 v;
                v.x = f32x2_to_bf16x2_rne(h[0], h[1]);
                v.y = f32x2_to_bf16x2_rne(h[2], h[3]);
                *reinterpret_cast<u32x2*>(stage + st_off(r, cb)) = v;
              } else {
                *reinterpret_cast<f32x4*>(stage + st_off(r, cb)) = f32x4{h[0], h[1], h[2], h[3]};
              }
            }
          }
        }
      }
      __syncthreads();
      for (int idx = tid; idx < PROWS * CPR; idx += kThreads) {
        const int r = idx / CPR, c = idx - r * CPR;
        const int lr = pass * PROWS + r;
        const int64_t col = col0 + c * (16 / OUT_ES);
        if (lr < rows && col < N) {
          u32x4* dst =
              reinterpret_cast<u32x4*>(g.C + (static_cast<int64_t>(crow + lr) * N + col) * OUT_ES);
          const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * ROWB + ((c ^ (r & XM)) << 4));
          if (PHASE == 2 && g.stream_c)
            __builtin_nontemporal_store(v, dst);
          else
            *dst = v;
        }
      }
      if (pass + 1 < PASSES) __syncthreads();
    }
  }

}

template <int DT, int PHASE, int BM, int BN, int WM, int WN, int KRB_, int SCHED, bool WKN>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(GemmArgs g) {
  using G = Geo<DT, PHASE, BM, BN, WM, WN, KRB_>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // the task hand-over slot lives in the last bytes of the ring: it is
  // written after every wave is done with the ring and read before the
  // first DMA of the task can reach that stage slot
  int& s_task = *reinterpret_cast<int*>(lds + G::RING - 16);

  const int tid = threadIdx.x;
  const uint64_t clk0 = __builtin_amdgcn_s_memtime(), ref0 = __builtin_amdgcn_s_memrealtime();
  // (the clock reads are scalar-memory ops: wait for them here, so that no
  // scalar load stays in flight through the main loops, where it would force
  // every LDS wait there to wait for all LDS reads)
  wait_lgkmcnt0();

  // XCD-aware work queue.  Each workgroup reads the XCD it runs on from the
  // XCC_ID hardware register and shares that XCD's L2 with the workgroups
  // there.  The m-tiles are cut into chunks of group_m consecutive m-tiles
  // (from the host: about the m-tiles of one expert, at most 8); chunk c
  // belongs to XCD c % 8, whose workgroups take its tasks n-tile by n-tile,
  // so the weight rows of an n-tile are shared by the concurrent m-tiles of
  // the chunk and the activation rows of an m-tile by the n-tiles in flight
  // -- in one L2.  A drained XCD queue makes its workgroups steal from the
  // others, so the queue stays work-conserving under routing skew.
  const TaskQueue q{g.tm.queue + kXcd * g.queue_idx, *g.tm.n_mtiles, g.n_tiles_n, g.group_m,
                    (*g.tm.n_mtiles + g.group_m - 1) / g.group_m,
                    // s_getreg_b32 hwreg(HW_REG_XCC_ID, 0, 4): id of this XCD
                    static_cast<int>(__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) &
                                     (kXcd - 1)),
                    g.queue_order};
  const int NT = q.NT;
  const int own_limit = q.limit(q.xcd);
  bool own_open = true;  // (thread 0) the own XCD queue may still hold tasks

  if (tid == 0) s_task = q.pull(0);
  __syncthreads();
  for (;;) {
    const int task = __builtin_amdgcn_readfirstlane(s_task);
    if (task < 0) break;
    // The next task is requested from the own XCD queue while this one runs:
    // one atomic issued a few k-steps before the end, its result used after
    // the epilogue.  That hides the queue round trip behind the tile's last
    // k-steps while keeping the reservation short, so that the tail of the
    // queue still spreads over all workgroups.
    int next_v = -1;
    const int mt = task / NT;
    const int nt = task - mt * NT;
    uint64_t t_start = 0;
    if (g.task_log) {
      t_start = __builtin_amdgcn_s_memrealtime();
      wait_lgkmcnt0();
    }
    gemm_task<DT, PHASE, BM, BN, WM, WN, KRB_, SCHED, WKN>(
        g, mt, nt, -1, -1,
        [&] {
          if (tid == 0 && own_open) next_v = atomicAdd(&q.counters[q.xcd], 1);
        },
        [] {});

    // hand over the next task; the barriers also separate this task's last
    // LDS reads from the hand-over slot write and from the next task's
    // first DMA writes
    __syncthreads();
    if (tid == 0 && g.task_log && task < g.task_log_capacity) {
      // debug record of this task: start and end on the 100 MHz chip-wide
      // reference clock, the workgroup and the XCD that ran it
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      uint32_t* r = g.task_log + 4ll * task;
      r[0] = static_cast<uint32_t>(t_start);
      r[1] = static_cast<uint32_t>(t_end - t_start);
      r[2] = blockIdx.x;
      r[3] = static_cast<uint32_t>(q.xcd) | 0x100u;
    }
    if (tid == 0) {
      int t = -1;
      if (next_v >= 0) {
        if (next_v < own_limit) t = q.decode(next_v, q.xcd);
        else own_open = false;
      }
      if (t < 0) t = q.pull(own_open ? 0 : 1);
      s_task = t;
    }
    __syncthreads();
  }
  // sustained-clock record of the first workgroup (it lives as long as the
  // launch): shader-clock and 100 MHz reference ticks
  if (g.clock && blockIdx.x == 0 && tid == 0) {
    const uint64_t clk = __builtin_amdgcn_s_memtime() - clk0;
    const uint64_t ref = __builtin_amdgcn_s_memrealtime() - ref0;
    g.clock[0] = clk;
    g.clock[1] = ref;
  }
}

// ---------------------------------------------------------------------------
// Single-launch pipeline: W1/W3 and W2 tasks in one persistent grid, h passed
// through a bounded ring with full / empty counters per chunk (the ring of
// in-flight blocks and the L1/L2 full and empty counters of the
// MegaMoE-vs-MoE-systems page, sections 2.3 and 2.7).  h crosses XCDs (a
// W1/W3 task may be stolen by another XCD), so the full count is published
// with an agent-scope release after the h stores and awaited with an
// agent-scope acquire before the W2 task's first h load: the L2 write-back
// and invalidation those imply are what makes h coherent across the per-XCD
// L2s.  Waits are bounded: a wait that exceeds RingArgs::poll_limit polls
// gives up, sets RingArgs::err and lets the task run on (its output is then
// wrong, never a hang).  RingArgs::unreachable lifts every target beyond any
// count, so that the caller can exercise that failure report.
__device__ inline void ring_wait(int32_t* cnt, int need, bool acquire, int32_t* err, int limit) {
  for (int it = 0;; ++it) {
    const int v = acquire ? __hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
                          : __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= need) return;
    if (it >= limit) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void ring_gemm_kernel(GemmArgs g1, GemmArgs g2,
                                                                 RingArgs r) {
  using G1 = Geo<kBF16, 1, BM, BN, WM, WN, 128>;
  using G2 = Geo<kBF16, 2, BM, BN, WM, WN, 128>;
  static_assert(G1::RING == G2::RING, "one LDS ring for both phases");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int& s_task = *reinterpret_cast<int*>(lds + G1::RING - 16);  // as in grouped_gemm_kernel
  const int tid = threadIdx.x;
  const int M = *g1.tm.n_mtiles, GM = g1.group_m, NT1 = g1.n_tiles_n, NT2 = g2.n_tiles_n;
  const int nchunks = (M + GM - 1) / GM;
  const int xcd = static_cast<int>(__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) &
                                   (kXcd - 1));
  const int per_step = GM * (NT1 + NT2);
  auto owned = [&](int y) { return nchunks > y ? (nchunks - y + kXcd - 1) / kXcd : 0; };
  auto limit = [&](int y) { return (owned(y) + kRingLag) * per_step; };
  // pull v of queue y -> (phase, chunk index j of that queue, m-tile, n-tile);
  // false for a hole (no such chunk, or past the last m-tile)
  auto decode = [&](int v, int y, int& phase, int& j, int& mt, int& nt) {
    const int st = v / per_step, p = v - st * per_step;
    int ml;
    if (p < GM * NT1) {
      phase = 1;
      j = st;
      ml = p % GM;
      nt = p / GM;
    } else {
      phase = 2;
      j = st - kRingLag;
      ml = (p - GM * NT1) % GM;
      nt = (p - GM * NT1) / GM;
    }
    if (j < 0 || j >= owned(y)) return false;
    mt = (y + kXcd * j) * GM + ml;
    return mt < M;
  };
  // task codes: (queue << 24) | pull index
  auto pull = [&](int s0) {
    for (int s = s0; s < kXcd; ++s) {
      const int y = (xcd + s) % kXcd;
      const int lim = limit(y);
      for (;;) {
        if (__hip_atomic_load(&r.queue[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= lim)
          break;
        const int v = atomicAdd(&r.queue[y], 1);
        if (v >= lim) break;
        int ph, j, mt, nt;
        if (decode(v, y, ph, j, mt, nt)) return (y << 24) | v;
      }
    }
    return -1;
  };
  bool own_open = true;
  if (tid == 0) s_task = pull(0);
  __syncthreads();
  for (;;) {
    const int code = __builtin_amdgcn_readfirstlane(s_task);
    if (code < 0) break;
    const int y = code >> 24;
    int phase, j, mt, nt;
    decode(code & 0xffffff, y, phase, j, mt, nt);
    const int c = y + kXcd * j;  // chunk of the tile map
    const int64_t ring_row =
        (static_cast<int64_t>(y * r.slots + j % r.slots) * GM + (mt - c * GM)) * BM;
    int next_v = -1;
    auto kpull = [&] {
      if (tid == 0 && own_open) next_v = atomicAdd(&r.queue[xcd], 1);
    };
    if (phase == 1) {
      // before the h stores: the W2 tasks of the chunk that used this ring
      // slot before (slots steps earlier in the same queue) are all done
      auto slot_free = [&] {
        if (j >= r.slots) {
          const int cp = y + kXcd * (j - r.slots);
          if (tid == 0)
            ring_wait(&r.l2_done[cp], min(GM, M - cp * GM) * NT2 + r.unreachable, false, r.err,
                      r.poll_limit);
          __syncthreads();
        }
      };
      gemm_task<kBF16, 1, BM, BN, WM, WN, 128, 0, false>(g1, mt, nt, -1, ring_row, kpull,
                                                        slot_free);
      wait_vmcnt(0);  // this wave's h stores are done
      __syncthreads();
      if (tid == 0)
        __hip_atomic_fetch_add(&r.l1_done[c], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // every W1/W3 task of the chunk has published its h columns
      if (tid == 0)
        ring_wait(&r.l1_done[c], min(GM, M - c * GM) * NT1 + r.unreachable, true, r.err,
                  r.poll_limit);
      __syncthreads();
      gemm_task<kBF16, 2, BM, BN, WM, WN, 128, 0, false>(g2, mt, nt, ring_row, -1, kpull, [] {});
      __syncthreads();  // (the task's h loads all landed before its last stage)
      if (tid == 0) __hip_atomic_fetch_add(&r.l2_done[c], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // hand over the next task
    __syncthreads();
    if (tid == 0) {
      int t = -1;
      if (next_v >= 0) {
        int ph, jj, m2, n2;
        if (next_v < limit(xcd)) {
          if (decode(next_v, xcd, ph, jj, m2, n2)) t = (xcd << 24) | next_v;
        } else {
          own_open = false;
        }
      }
      if (t < 0) t = pull(own_open ? 0 : 1);
      s_task = t;
    }
    __syncthreads();
  }
}

template <int DT, int PHASE, int BM, int BN, int WM, int WN, int KRB = (DT == kF32 ? 64 : 128),
          int SCHED = 0, bool WKN = false>
struct Variant {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int lds_bytes() { return Geo<DT, PHASE, BM, BN, WM, WN, KRB>::LDS; }
  static int launch(const GemmArgs& a, hipStream_t s) {
    auto kern = grouped_gemm_kernel<DT, PHASE, BM, BN, WM, WN, KRB, SCHED, WKN>;
    static int grid = 0;
    static hipError_t attr_err = hipSuccess;
    static std::once_flag once;
    std::call_once(once, [&] {
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes());
      int dev = 0, cus = 0, per_cu = 0;
      (void)hipGetDevice(&dev);
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds_bytes());
      grid = max(1, cus) * max(1, per_cu);
    });
    if (attr_err != hipSuccess) return static_cast<int>(attr_err);
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
#define MOE_V(DT, P, BM_, VAR, BN_, WM_, WN_, ...)                \
  if (dtype == DT && phase == P && bm == BM_ && var == VAR)        \
    return f(Variant<DT, P, BM_, BN_, WM_, WN_ __VA_OPT__(, ) __VA_ARGS__>{});
  // SCHED bit 4: MFMAs of the padding rows skipped per wave (2.09 against
  // 2.14 ms on the skewed layer, 17.49 against 17.54 ms on the FP8 one);
  // bit 3: W2 stores its fp16 Y from registers (W2 0.682 against 0.696 ms
  // on the skewed layer, 0.292 against 0.2975 on the prefill one)
  MOE_V(kBF16, 1, 256, 0, 256, 2, 4, 128, 16)
  MOE_V(kBF16, 2, 256, 0, 256, 2, 4, 128, 24)
  // measured alternatives of the 256 x 256 schedule (slower, or no faster,
  // on the prefill and skewed layers): 3 = DMA interleaved with the MFMAs,
  // 4 = ping-pong of the two waves of each SIMD, 5 = the second k-step's
  // fragments read during the first one's MFMAs, 6 = every fragment row's
  // MFMAs run, 7 = W2's Y staged through LDS, 8 = h stored from registers
  // (no gain on the bf16 layers)
  MOE_V(kBF16, 1, 256, 3, 256, 2, 4, 128, 2)
  MOE_V(kBF16, 2, 256, 3, 256, 2, 4, 128, 2)
  MOE_V(kBF16, 1, 256, 4, 256, 2, 4, 128, 1)
  MOE_V(kBF16, 2, 256, 4, 256, 2, 4, 128, 1)
  MOE_V(kBF16, 1, 256, 5, 256, 2, 4, 128, 4)
  MOE_V(kBF16, 2, 256, 5, 256, 2, 4, 128, 4)
  MOE_V(kBF16, 1, 256, 6, 256, 2, 4)
  MOE_V(kBF16, 2, 256, 6, 256, 2, 4)
  MOE_V(kBF16, 1, 256, 8, 256, 2, 4, 128, 24)
  MOE_V(kBF16, 2, 256, 7, 256, 2, 4, 128, 16)
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
  // FP8 W1/W3 stores its h codes from registers (9.02 against 9.11 ms)
  MOE_V(kFP8, 1, 256, 0, 256, 2, 4, 128, 24)
  MOE_V(kFP8, 2, 256, 0, 256, 2, 4, 128, 24)
  MOE_V(kFP8, 1, 256, 6, 256, 2, 4)
  MOE_V(kFP8, 2, 256, 6, 256, 2, 4)
  MOE_V(kFP8, 1, 256, 8, 256, 2, 4, 128, 16)
  MOE_V(kFP8, 2, 256, 7, 256, 2, 4, 128, 16)
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
  MOE_V(kMX4, 1, 256, 0, 256, 2, 4)
  MOE_V(kMX4, 2, 256, 0, 256, 2, 4)
  MOE_V(kMX4, 1, 128, 0, 256, 2, 4)
  MOE_V(kMX4, 2, 128, 0, 256, 2, 4)
  MOE_V(kMX4, 1, 64, 0, 256, 1, 4)
  MOE_V(kMX4, 2, 64, 0, 256, 1, 4)
  MOE_V(kMX4, 1, 32, 0, 256, 1, 4)
  MOE_V(kMX4, 2, 32, 0, 256, 1, 4)
  MOE_V(kMX4, 1, 16, 0, 256, 1, 4)
  MOE_V(kMX4, 2, 16, 0, 256, 1, 4)
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

// Kernel with k-row weight tiles (the stated [K][N] weight layout) per
// (dtype, phase, tile height): the default shapes.
template <typename F>
int dispatch_kn(int phase, int dtype, int bm, F&& f) {
#define MOE_KN(DT, P, BM_, BN_, WM_, WN_, ...)                                        \
  if (dtype == DT && phase == P && bm == BM_)                                        \
    return f(Variant<DT, P, BM_, BN_, WM_, WN_, (DT == kF32 ? 64 : 128),             \
                     0 __VA_OPT__(| __VA_ARGS__), true>{});
  MOE_KN(kBF16, 1, 256, 256, 2, 4)
  MOE_KN(kBF16, 2, 256, 256, 2, 4)
  MOE_KN(kBF16, 1, 128, 128, 2, 2)
  MOE_KN(kBF16, 2, 128, 128, 2, 2)
  MOE_KN(kBF16, 1, 64, 128, 1, 4)
  MOE_KN(kBF16, 2, 64, 128, 1, 4)
  MOE_KN(kBF16, 1, 32, 128, 1, 4)
  MOE_KN(kBF16, 2, 32, 128, 1, 4)
  MOE_KN(kBF16, 1, 16, 256, 1, 4)
  MOE_KN(kBF16, 2, 16, 256, 1, 4)
  MOE_KN(kFP8, 1, 256, 256, 2, 4)
  MOE_KN(kFP8, 2, 256, 256, 2, 4)
  MOE_KN(kFP8, 1, 128, 256, 2, 4)
  MOE_KN(kFP8, 2, 128, 256, 2, 4)
  MOE_KN(kFP8, 1, 64, 256, 1, 4)
  MOE_KN(kFP8, 2, 64, 128, 1, 4)
  MOE_KN(kFP8, 1, 32, 256, 2, 2)
  MOE_KN(kFP8, 2, 32, 128, 1, 4)
  MOE_KN(kFP8, 1, 16, 256, 1, 4)
  MOE_KN(kFP8, 2, 16, 128, 1, 4)
  MOE_KN(kF32, 1, 256, 128, 2, 2)
  MOE_KN(kF32, 2, 256, 128, 2, 2)
  MOE_KN(kF32, 1, 128, 128, 2, 2)
  MOE_KN(kF32, 2, 128, 128, 2, 2)
  MOE_KN(kF32, 1, 64, 128, 1, 4)
  MOE_KN(kF32, 2, 64, 128, 1, 4)
  MOE_KN(kF32, 1, 32, 128, 1, 4)
  MOE_KN(kF32, 2, 32, 128, 1, 4)
  MOE_KN(kF32, 1, 16, 128, 1, 4)
  MOE_KN(kF32, 2, 16, 128, 1, 4)
#undef MOE_KN
  return -1;
}

template <typename F>
int dispatch(int phase, int dtype, int bm, bool wkn, F&& f) {
  if (wkn) return dispatch_kn(phase, dtype, bm, f);
  int r = dispatch_var(phase, dtype, bm, variant_choice(), f);
  if (r == -1 && variant_choice() != 0) r = dispatch_var(phase, dtype, bm, 0, f);
  return r;
}

}  // namespace

int launch_gemm(int phase, int dtype, int bm, bool wkn, const GemmArgs& a, hipStream_t s) {
  return dispatch(phase, dtype, bm, wkn, [&](auto v) { return decltype(v)::launch(a, s); });
}

int gemm_tile_n(int phase, int dtype, int bm, bool wkn) {
  return dispatch(phase, dtype, bm, wkn, [&](auto v) { return decltype(v)::tile_n(); });
}

int launch_gemm_ring(const GemmArgs& g1, const GemmArgs& g2, const RingArgs& r, hipStream_t s) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
  using G1 = Geo<kBF16, 1, BM, BN, WM, WN, 128>;
  using G2 = Geo<kBF16, 2, BM, BN, WM, WN, 128>;
  constexpr int lds = G1::LDS > G2::LDS ? G1::LDS : G2::LDS;
  auto kern = ring_gemm_kernel<BM, BN, WM, WN>;
  static int grid = 0;
  static hipError_t attr_err = hipSuccess;
  static std::once_flag once;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WM * WN * 64, lds);
    grid = max(1, cus) * max(1, per_cu);
  });
  if (attr_err != hipSuccess) return static_cast<int>(attr_err);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WM * WN * 64), lds, s, g1, g2, r);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
