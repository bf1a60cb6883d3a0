// api.cpp -- the C ABI of libmoe.so: argument checks, workspace layout and
// the launch sequence of the layer forward.  See include/moe.h for the
// contract of every entry point.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local int g_last_hip = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int esize(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }

// Bytes of a [rows x cols] expert-weight matrix in w_dtype (FP4: two per byte).
int64_t weight_matrix_bytes(int dt, int64_t rows, int64_t cols) {
  return dt == MOE_MXFP4 ? rows * cols / 2 : rows * cols * esize(dt);
}

bool quantised_weights(int dt) { return dt == MOE_FP8_E4M3 || dt == MOE_MXFP4; }

// Tile height from the expected rows per expert, T*k/E: the serving-regime
// choice of the MegaMoE-vs-MoE-systems page (section 2.5), re-tuned for
// 16-row MFMA fragments and four 64-wide waves per workgroup.
int pick_bm(const moe_problem& p) {
  if (p.block_m) return p.block_m;
  const double r = static_cast<double>(p.T) * p.top_k / p.E;
  if (r <= 24.0) return 16;
  if (r <= 48.0) return 32;
  if (r <= 160.0) return 64;
  if (r < 384.0) return 128;
  return 256;
}

// m-tiles per XCD work chunk: about the m-tiles one expert fills (so the
// expert's weight tiles are reused by all of them at once), between 1 and 8;
// MOE_GROUP_M overrides it for tuning.
int group_m(const moe_problem& p, int bm) {
  static const int forced = [] {
    const char* e = getenv("MOE_GROUP_M");
    return e ? atoi(e) : 0;
  }();
  if (forced > 0) return std::min(forced, 8);
  const double r = static_cast<double>(p.T) * p.top_k / p.E / bm;
  const int gm = static_cast<int>(r + 0.999);
  return std::max(1, std::min(8, gm));
}

bool valid_problem(const moe_problem* p) {
  if (!p) return false;
  if (p->T < 0 || p->d <= 0 || p->f <= 0) return false;
  if (p->E < 1 || p->E > 1024 || p->top_k < 1 || p->top_k > p->E) return false;
  if (p->n_shared < 0 || p->n_shared > 8) return false;
  if (p->T > (1ll << 31) / 1024 || p->T * (p->top_k + p->n_shared) > (1ll << 30)) return false;
  const bool ok_types = (p->act_dtype == MOE_F32 && p->w_dtype == MOE_F32) ||
                        (p->act_dtype == MOE_BF16 && p->w_dtype == MOE_BF16) ||
                        (p->act_dtype == MOE_BF16 && p->w_dtype == MOE_FP8_E4M3) ||
                        (p->act_dtype == MOE_BF16 && p->w_dtype == MOE_MXFP4);
  if (!ok_types) return false;
  if (p->out_dtype != MOE_F32 && p->out_dtype != MOE_BF16) return false;
  if (p->block_m != 0 && p->block_m != 16 && p->block_m != 32 && p->block_m != 64 &&
      p->block_m != 128 && p->block_m != 256)
    return false;
  if (p->w_layout != MOE_W_KN && p->w_layout != MOE_W_NK) return false;
  return true;
}

// Weight layouts the GEMM kernels read: [N][K] (packed) for every dtype, and
// the stated [K][N] for F32, BF16 and FP8 weights (k-row weight tiles read
// with transposing LDS loads); MXFP4 codes are packed K-major by definition.
bool supported_layout(const moe_problem& p) {
  return p.w_layout == MOE_W_NK || p.w_dtype != MOE_MXFP4;
}

// Format of Y, the expert outputs per slot: fp32 on fp32 layers; bf16 for
// MXFP4 weights (their 5e-2 tolerance leaves room for the rounding); on bf16
// and FP8 layers fp16 codes under a power-of-two scale per 32 columns (one
// exponent byte per group, in its own region).  Y is the largest buffer of
// the layer and the combine's whole stream; an 11-bit significand keeps its
// rounding at most 2^-12 of each term, far inside either tolerance.
int y_format(const moe_problem& p) {
  if (p.w_dtype == MOE_MXFP4) return moe::kYBF16;
  if (p.w_dtype == MOE_FP8_E4M3 || p.act_dtype == MOE_BF16) return moe::kYF16E;
  return moe::kYF32;
}
int y_bytes(const moe_problem& p) { return y_format(p) == moe::kYF32 ? 4 : 2; }

// Floats per row of the FP8 activation scales inside the workspace (x and
// h: one per 128 elements): padded to a multiple of 4, so that the GEMM
// fetches four stages' scales of a row with one 16-byte load.
int64_t fp8_scale_stride(int64_t k) { return (k / 128 + 3) / 4 * 4; }

// Expert rows of the grouped GEMMs: the T*k routed slots, then T per shared
// expert.
int64_t gemm_rows(const moe_problem& p) { return p.T * (p.top_k + p.n_shared); }

// Shapes the kernels support (valid but unsupported -> MOE_ERR_UNSUPPORTED):
// contraction rows of 128 bytes, and every GEMM operand addressable with
// 32-bit byte offsets (x or its FP8 codes, h, one expert's weight matrix).
bool supported_shape(const moe_problem* p) {
  const int64_t m = p->w_dtype == MOE_F32 ? 32 : (p->w_dtype == MOE_BF16 ? 64 : 128);
  if (p->d % m != 0 || p->f % m != 0) return false;
  // activation element bytes of the GEMM operands (FP8 and MX FP8: 1)
  const int64_t es = p->w_dtype == MOE_F32 ? 4 : (p->w_dtype == MOE_BF16 ? 2 : 1);
  const int64_t lim = 1ll << 31;
  // FP8: the GEMMs stage a tile's weight block scales for the whole
  // contraction in LDS (at most kWscMax blocks of 128)
  if (p->w_dtype == MOE_FP8_E4M3 &&
      (p->d / 128 > moe::kWscMax || p->f / 128 > moe::kWscMax))
    return false;
  return p->T * p->d * es < lim && gemm_rows(*p) * p->f * es < lim &&
         weight_matrix_bytes(p->w_dtype, p->d, p->f) < lim;
}

struct Layout {
  size_t logits, ids, w, table, counts, offsets, slot_token, slot_k, token_slot;
  size_t tm_e, tm_row0, tm_rows, tm_misc;
  size_t xq, sx, hs, h, y, ye;
  size_t ring_ctrl;  // ring layout: queue[8], l1_done[max_mtiles], l2_done[max_mtiles], err
  size_t total;
  int bm;
  int64_t max_mtiles;
};

// Ring slots per XCD of the single-launch pipeline: chunk j's h waits in slot
// j % kRingSlots until its W2 tasks (kRingLag steps of the queue later) are
// done; the chunk that reuses the slot must come after them in the queue, so
// the slots must outnumber the lag.
constexpr int kRingSlots = 3;
static_assert(kRingSlots > moe::kRingLag, "slot reuse waits on earlier tasks only");
int64_t ring_ctrl_words(int64_t max_mtiles) { return 8 + 2 * max_mtiles + 1; }

Layout make_layout(const moe_problem& p, bool ring = false) {
  Layout L{};
  const int64_t n = p.T * p.top_k;
  const int64_t nchunk = ceil_div(n, moe::permute_chunk(n));
  const int64_t rows = gemm_rows(p);
  L.bm = pick_bm(p);
  L.max_mtiles = (n + static_cast<int64_t>(p.E) * (L.bm - 1)) / L.bm + 1 +
                 static_cast<int64_t>(p.n_shared) * ceil_div(p.T, L.bm);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + std::max<size_t>(bytes, 1));
    return at;
  };
  L.logits = take(sizeof(float) * p.T * p.E);
  L.ids = take(sizeof(int32_t) * n);
  L.w = take(sizeof(float) * n);
  L.table = take(sizeof(int32_t) * nchunk * p.E);
  L.counts = take(sizeof(int32_t) * p.E);
  L.offsets = take(sizeof(int32_t) * (p.E + 1));
  L.slot_token = take(sizeof(int32_t) * rows);
  L.slot_k = take(sizeof(int32_t) * rows);
  L.token_slot = take(sizeof(int32_t) * n);
  L.tm_e = take(sizeof(int32_t) * L.max_mtiles);
  L.tm_row0 = take(sizeof(int32_t) * L.max_mtiles);
  L.tm_rows = take(sizeof(int32_t) * L.max_mtiles);
  L.tm_misc = take(sizeof(int32_t) * (1 + moe::kQueueWords));
  const bool fp8 = p.w_dtype == MOE_FP8_E4M3, mx = p.w_dtype == MOE_MXFP4;
  // FP8: fp32 scales per 128 elements; MX: one E8M0 byte per 32 elements
  L.xq = take(fp8 || mx ? static_cast<size_t>(p.T) * p.d : 0);
  L.sx = take(fp8 ? sizeof(float) * p.T * fp8_scale_stride(p.d) : (mx ? p.T * (p.d / 32) : 0));
  L.hs = take(fp8 ? sizeof(float) * rows * fp8_scale_stride(p.f) : (mx ? rows * (p.f / 32) : 0));
  if (ring)  // h only for the chunks in flight: 8 XCDs x kRingSlots x group_m tiles
    L.h = take(static_cast<size_t>(8 * kRingSlots) * group_m(p, L.bm) * L.bm * p.f *
               esize(p.act_dtype));
  else
    L.h = take(static_cast<size_t>(rows) * p.f * (fp8 || mx ? 1 : esize(p.act_dtype)));
  L.y = take(static_cast<size_t>(y_bytes(p)) * rows * p.d);
  L.ye = take(y_format(p) == moe::kYF16E ? static_cast<size_t>(rows) * (p.d / 32) : 0);
  L.ring_ctrl = take(ring ? sizeof(int32_t) * ring_ctrl_words(L.max_mtiles) : 0);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

moe::TileMap tile_map(void* ws, const Layout& L) {
  moe::TileMap tm;
  tm.e = at<int32_t>(ws, L.tm_e);
  tm.row0 = at<int32_t>(ws, L.tm_row0);
  tm.rows = at<int32_t>(ws, L.tm_rows);
  tm.n_mtiles = at<int32_t>(ws, L.tm_misc);
  tm.queue = at<int32_t>(ws, L.tm_misc) + 1;
  return tm;
}

moe_status hip_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip = static_cast<int>(e);
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status from_code(int code) {
  if (code != 0) {
    g_last_hip = code;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// Workspace of moe_forward_noalloc: a device array of the library, one copy
// per GPU (each device's copy has its own address), held until the process
// ends.  Host code never passes `scratch` itself to a kernel or a copy -- on
// the host it only names the symbol; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = MOE_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the calling thread's current device's scratch array.
moe_status scratch_of_current_device(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_code(static_cast<int>(e));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return from_code(static_cast<int>(g_scratch_err[dev]));
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or type combination";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEVICE: return "a bounded wait inside a launch gave up";
  }
  return "unknown status";
}

int moe_last_hip_error(void) { return g_last_hip; }

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
  if (!valid_problem(p) || !bytes) return MOE_ERR_INVALID_ARG;
  *bytes = make_layout(*p).total;
  return MOE_OK;
}

moe_status moe_weight_bytes(const moe_problem* p, size_t* bytes) {
  if (!valid_problem(p) || !bytes) return MOE_ERR_INVALID_ARG;
  *bytes = static_cast<size_t>((p->E + p->n_shared) * weight_matrix_bytes(p->w_dtype, p->d, p->f));
  return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const void* x, const void* gate_w, const float* bias,
                     float* logits, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (!valid_problem(p)) return MOE_ERR_INVALID_ARG;
  if (p->d % 32 != 0) return MOE_ERR_UNSUPPORTED;  // hidden chunks of 32 in the gate
  if (p->T == 0) return MOE_OK;
  if (!x || !gate_w || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  float* lg = logits;
  if (!lg) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(*p);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    lg = at<float>(ws, L.logits);
  }
  (void)hipGetLastError();
  return from_code(moe::launch_gate(x, gate_w, bias, lg, topk_ids, topk_w,
                                    static_cast<int>(p->T), static_cast<int>(p->d), p->E,
                                    p->top_k, p->act_dtype == MOE_BF16, stream));
}

moe_status moe_permute(const moe_problem* p, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* slot_token, int32_t* slot_k,
                       int32_t* token_slot, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_problem(p)) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets || !ws) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!topk_ids || !slot_token || !slot_k || !token_slot))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*p);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  (void)hipGetLastError();
  moe::launch_permute(topk_ids, static_cast<int>(p->T), p->top_k, p->E, 0, L.bm,
                      at<int32_t>(ws, L.table), counts, offsets, slot_token, slot_k, token_slot,
                      tile_map(ws, L), stream);
  return hip_status();
}

moe_status moe_quantize_fp8(int64_t rows, int64_t cols, const void* x_bf16, uint8_t* q,
                            float* s, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x_bf16 || !q || !s) return MOE_ERR_INVALID_ARG;
  (void)hipGetLastError();
  moe::launch_quant_fp8(static_cast<const uint16_t*>(x_bf16), rows, cols, q, s, cols / 128,
                        stream);
  return hip_status();
}

moe_status moe_quantize_mx(int64_t rows, int64_t cols, const void* x_bf16, uint8_t* q,
                           uint8_t* s, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x_bf16 || !q || !s) return MOE_ERR_INVALID_ARG;
  (void)hipGetLastError();
  moe::launch_quant_mx(static_cast<const uint16_t*>(x_bf16), rows, cols, q, s, stream);
  return hip_status();
}

moe_status moe_pack_weight(int32_t E, int64_t K, int64_t N, int32_t elem_bytes, const void* src,
                           void* dst, hipStream_t stream) {
  if (E < 1 || K < 1 || N < 1 || !src || !dst) return MOE_ERR_INVALID_ARG;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return MOE_ERR_INVALID_ARG;
  // one workgroup per 64 x 64 tile: K / 64 and E index the grid's y and z
  // dimensions (at most 65535 each)
  if (K > 65535ll * 64 || N > (1ll << 24) || E > 65535) return MOE_ERR_UNSUPPORTED;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t len = static_cast<uintptr_t>(E) * K * N * elem_bytes;
  if (a < b + len && b < a + len) return MOE_ERR_INVALID_ARG;  // overlap
  (void)hipGetLastError();
  moe::launch_pack(E, K, N, elem_bytes, src, dst, stream);
  return hip_status();
}

}  // extern "C"

namespace {

// The single-launch pipeline covers bf16 layers with 256-row tiles (and task
// codes below 2^24: queue << 24 | pull index).
bool ring_supported(const moe_problem& p) {
  if (p.act_dtype != MOE_BF16 || p.w_dtype != MOE_BF16 || pick_bm(p) != 256) return false;
  if (p.w_layout != MOE_W_NK) return false;
  const int64_t gm = group_m(p, 256);
  const int64_t tiles = (gemm_rows(p) + static_cast<int64_t>(p.E + p.n_shared) * 255) / 256 + 1;
  const int64_t per_step = gm * (ceil_div(2 * p.f, 256) + ceil_div(p.d, 256));
  return (ceil_div(ceil_div(tiles, gm), 8) + moe::kRingLag) * per_step < (1ll << 24);
}

moe_status forward_impl(const moe_problem* p, const void* x, const void* gate_w,
                        const float* bias, const void* W1t, const void* W3t, const void* W2t,
                        const void* W1s, const void* W3s, const void* W2s, void* out, void* ws,
                        size_t ws_bytes, const moe_debug* dbg, hipStream_t stream, bool ring) {
  if (!valid_problem(p)) return MOE_ERR_INVALID_ARG;
  if (!supported_shape(p) || !supported_layout(*p)) return MOE_ERR_UNSUPPORTED;
  if (ring && !ring_supported(*p)) return MOE_ERR_UNSUPPORTED;
  if (dbg && (dbg->queue_order < 0 || dbg->queue_order > 2 || dbg->task_log_capacity < 0 ||
              (dbg->task_log && dbg->task_log_capacity == 0)))
    return MOE_ERR_INVALID_ARG;
  if (ring && dbg) {
    if (dbg->ring_poll_limit < 0) return MOE_ERR_INVALID_ARG;
    if (dbg->ring_force_timeout &&
        (dbg->ring_poll_limit < 1 || dbg->ring_poll_limit > moe::kRingForcedPollMax))
      return MOE_ERR_INVALID_ARG;
  }
  if (p->T == 0) return MOE_OK;
  if (!x || !gate_w || !W1t || !W3t || !W2t || !out || !ws) return MOE_ERR_INVALID_ARG;
  const bool fp8 = p->w_dtype == MOE_FP8_E4M3, mx = p->w_dtype == MOE_MXFP4;
  const bool q8 = fp8 || mx;  // the GEMMs read 1-byte activation codes + scales
  if (q8 && (!W1s || !W3s || !W2s)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*p, ring);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  const int T = static_cast<int>(p->T), d = static_cast<int>(p->d);
  const int E = p->E, k = p->top_k;
  const int n = T * k;
  float* logits = at<float>(ws, L.logits);
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* w = at<float>(ws, L.w);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* slot_token = at<int32_t>(ws, L.slot_token);
  int32_t* slot_k = at<int32_t>(ws, L.slot_k);
  int32_t* token_slot = at<int32_t>(ws, L.token_slot);
  const moe::TileMap tm = tile_map(ws, L);
  const int hdt = fp8 ? moe::kFP8
                      : (mx ? moe::kMX4 : (p->act_dtype == MOE_BF16 ? moe::kBF16 : moe::kF32));
  const int gdt = hdt;

  auto mark = [&](int i) {
    if (dbg && dbg->stage_events[i]) (void)hipEventRecord(dbg->stage_events[i], stream);
  };
  (void)hipGetLastError();
  mark(0);
  // 1. gate; on FP8 and MXFP4 layers it also quantises x (FP8 per 1x128
  // group, or MX FP8 per 32) in the same pass over x
  moe_status st = from_code(moe::launch_gate(
      x, gate_w, bias, logits, ids, w, T, d, E, k, p->act_dtype == MOE_BF16, stream,
      fp8 ? 1 : (mx ? 2 : 0), q8 ? at<uint8_t>(ws, L.xq) : nullptr,
      q8 ? at<void>(ws, L.sx) : nullptr, fp8_scale_stride(p->d)));
  if (st != MOE_OK) return st;
  mark(1);
  mark(2);  // (stage 2, the activation quantisation, is inside the gate)
  // 3. histogram, scan + tile map, scatter
  moe::launch_permute(ids, T, k, E, p->n_shared, L.bm, at<int32_t>(ws, L.table), counts,
                      offsets, slot_token, slot_k, token_slot, tm, stream);
  mark(3);
  st = hip_status();
  if (st != MOE_OK) return st;

  // 4. W1/W3 + SwiGLU
  moe::GemmArgs g1{};
  g1.A = q8 ? at<uint8_t>(ws, L.xq) : static_cast<const uint8_t*>(x);
  g1.a_row_bytes = p->d * (q8 ? 1 : esize(p->act_dtype));
  g1.a_bytes = p->T * g1.a_row_bytes;
  g1.gather = slot_token;
  g1.sa = q8 ? at<float>(ws, L.sx) : nullptr;  // (MX: E8M0 bytes)
  g1.sa_stride = static_cast<int>(fp8_scale_stride(p->d));
  g1.sa_bytes = fp8 ? static_cast<int64_t>(L.hs - L.sx) : 0;  // the x scale region
  g1.B0 = static_cast<const uint8_t*>(W1t);
  g1.B1 = static_cast<const uint8_t*>(W3t);
  g1.sb0 = static_cast<const float*>(W1s);
  g1.sb1 = static_cast<const float*>(W3s);
  g1.K = p->d;
  g1.N = p->f;
  g1.C = at<uint8_t>(ws, L.h);
  g1.sc = q8 ? at<float>(ws, L.hs) : nullptr;
  g1.sc_stride = static_cast<int>(fp8_scale_stride(p->f));
  g1.tm = tm;
  const bool wkn = p->w_layout == MOE_W_KN;
  g1.n_tiles_n = static_cast<int>(ceil_div(2 * p->f, moe::gemm_tile_n(1, gdt, L.bm, wkn)));
  g1.queue_idx = 0;
  g1.group_m = group_m(*p, L.bm);
  g1.clock = dbg ? dbg->gemm_clock : nullptr;
  g1.queue_order = dbg ? dbg->queue_order : 0;
  g1.task_log = dbg ? dbg->task_log : nullptr;
  g1.task_log_capacity = dbg ? dbg->task_log_capacity : 0;
  if (!ring) {
    st = from_code(moe::launch_gemm(1, gdt, L.bm, wkn, g1, stream));
    if (st != MOE_OK) return st;
    mark(4);
  }

  // 5. W2
  moe::GemmArgs g2{};
  g2.A = at<uint8_t>(ws, L.h);
  g2.a_row_bytes = p->f * (q8 ? 1 : esize(p->act_dtype));
  g2.a_bytes = static_cast<int64_t>(L.y - L.h);  // the h region
  g2.gather = nullptr;
  g2.sa = q8 ? at<float>(ws, L.hs) : nullptr;
  g2.sa_stride = static_cast<int>(fp8_scale_stride(p->f));
  g2.sa_bytes = fp8 ? static_cast<int64_t>(L.h - L.hs) : 0;  // the h scale region
  g2.B0 = static_cast<const uint8_t*>(W2t);
  g2.B1 = nullptr;
  g2.sb0 = static_cast<const float*>(W2s);
  g2.sb1 = nullptr;
  g2.K = p->f;
  g2.N = p->d;
  g2.C = at<uint8_t>(ws, L.y);
  g2.ce = y_format(*p) == moe::kYF16E ? at<uint8_t>(ws, L.ye) : nullptr;
  g2.sc = nullptr;
  g2.tm = tm;
  g2.n_tiles_n = static_cast<int>(ceil_div(p->d, moe::gemm_tile_n(2, gdt, L.bm, wkn)));
  g2.queue_idx = 1;
  g2.group_m = g1.group_m;
  // Y far larger than the 256 MB MALL is read back from HBM by the combine
  // anyway: non-temporal stores keep it from displacing the operands cached
  // for the GEMMs (measured 1-3 % on W2 and the combine for Y of 0.8-7.5 GB;
  // for a 268 MB Y the combine lost what W2 gained)
  g2.stream_c = static_cast<double>(gemm_rows(*p)) * p->d * y_bytes(*p) >= 512.0 * (1 << 20);
  g2.clock = (dbg && dbg->gemm_clock) ? dbg->gemm_clock + 2 : nullptr;
  g2.queue_order = g1.queue_order;
  g2.task_log = g1.task_log ? g1.task_log + 4ll * g1.task_log_capacity : nullptr;
  g2.task_log_capacity = g1.task_log_capacity;
  if (!ring) {
    st = from_code(moe::launch_gemm(2, gdt, L.bm, wkn, g2, stream));
    if (st != MOE_OK) return st;
  } else {
    // both GEMMs in one launch; h lives in the ring, Y in full
    moe::RingArgs r{};
    int32_t* ctrl = at<int32_t>(ws, L.ring_ctrl);
    r.h = at<uint8_t>(ws, L.h);
    r.queue = ctrl;
    r.l1_done = ctrl + 8;
    r.l2_done = ctrl + 8 + L.max_mtiles;
    r.err = ctrl + 8 + 2 * L.max_mtiles;
    r.slots = kRingSlots;
    r.poll_limit = (dbg && dbg->ring_poll_limit > 0) ? dbg->ring_poll_limit : moe::kRingPollLimit;
    r.unreachable = (dbg && dbg->ring_force_timeout) ? (1 << 30) : 0;
    g1.C = r.h;
    g2.A = r.h;
    g1.clock = g2.clock = nullptr;
    g1.task_log = g2.task_log = nullptr;  // (the ring kernel keeps no task log)
    g1.queue_order = g2.queue_order = 0;
    moe::launch_zero(ctrl, ring_ctrl_words(L.max_mtiles), stream);
    st = from_code(moe::launch_gemm_ring(g1, g2, r, stream));
    if (st != MOE_OK) return st;
    mark(4);
  }
  mark(5);

  // 6. combine
  moe::launch_combine(at<uint8_t>(ws, L.y), y_format(*p), at<uint8_t>(ws, L.ye), w, token_slot,
                      out, T, d, k,
                      p->n_shared, p->out_dtype == MOE_BF16, stream);
  mark(6);

  if (dbg) {
    auto cp = [&](void* dst, const void* src, size_t bytes) {
      if (dst) (void)hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream);
    };
    cp(dbg->topk_ids, ids, sizeof(int32_t) * n);
    cp(dbg->topk_w, w, sizeof(float) * n);
    cp(dbg->counts, counts, sizeof(int32_t) * E);
    cp(dbg->offsets, offsets, sizeof(int32_t) * (E + 1));
    cp(dbg->slot_token, slot_token, sizeof(int32_t) * n);
    cp(dbg->slot_k, slot_k, sizeof(int32_t) * n);
    cp(dbg->token_slot, token_slot, sizeof(int32_t) * n);
    if (q8) {
      cp(dbg->x_codes, at<uint8_t>(ws, L.xq), static_cast<size_t>(p->T) * p->d);
      if (dbg->x_scales && fp8)  // drop the row padding of the workspace copy
        (void)hipMemcpy2DAsync(dbg->x_scales, sizeof(float) * (p->d / 128), at<float>(ws, L.sx),
                               sizeof(float) * fp8_scale_stride(p->d),
                               sizeof(float) * (p->d / 128), p->T, hipMemcpyDeviceToDevice,
                               stream);
      if (mx) cp(dbg->x_scales, at<uint8_t>(ws, L.sx), static_cast<size_t>(p->T) * (p->d / 32));
    }
    if (!ring) {  // (the ring keeps only the chunks in flight)
      const int64_t rows = gemm_rows(*p);
      cp(dbg->h, at<uint8_t>(ws, L.h),
         static_cast<size_t>(rows) * p->f * (q8 ? 1 : esize(p->act_dtype)));
      if (dbg->h_scales && fp8)
        (void)hipMemcpy2DAsync(dbg->h_scales, sizeof(float) * (p->f / 128), at<float>(ws, L.hs),
                               sizeof(float) * fp8_scale_stride(p->f),
                               sizeof(float) * (p->f / 128), rows, hipMemcpyDeviceToDevice,
                               stream);
      if (mx) cp(dbg->h_scales, at<uint8_t>(ws, L.hs), static_cast<size_t>(rows) * (p->f / 32));
    }
  }
  return hip_status();
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_problem* p, const void* x, const void* gate_w, const float* bias,
                       const void* W1, const void* W3, const void* W2, const void* W1s,
                       const void* W3s, const void* W2s, void* out, void* ws, size_t ws_bytes,
                       const moe_debug* dbg, hipStream_t stream) {
  return forward_impl(p, x, gate_w, bias, W1, W3, W2, W1s, W3s, W2s, out, ws, ws_bytes, dbg,
                      stream, false);
}

moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* gate_w,
                               const float* bias, const void* W1, const void* W3, const void* W2,
                               const void* W1s, const void* W3s, const void* W2s, void* out,
                               const moe_debug* dbg, hipStream_t stream) {
  if (!valid_problem(p)) return MOE_ERR_INVALID_ARG;
  if (make_layout(*p).total > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const moe_status st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  return forward_impl(p, x, gate_w, bias, W1, W3, W2, W1s, W3s, W2s, out, ws, kScratchBytes, dbg,
                      stream, false);
}

moe_status moe_ring_workspace_size(const moe_problem* p, size_t* bytes) {
  if (!bytes || !valid_problem(p)) return MOE_ERR_INVALID_ARG;
  if (!supported_shape(p) || !ring_supported(*p)) return MOE_ERR_UNSUPPORTED;
  *bytes = make_layout(*p, true).total;
  return MOE_OK;
}

moe_status moe_ring_error_flag(const moe_problem* p, void* ws, size_t ws_bytes, int32_t** flag) {
  if (!flag || !ws || !valid_problem(p)) return MOE_ERR_INVALID_ARG;
  if (!supported_shape(p) || !ring_supported(*p)) return MOE_ERR_UNSUPPORTED;
  const Layout L = make_layout(*p, true);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  *flag = at<int32_t>(ws, L.ring_ctrl) + 8 + 2 * L.max_mtiles;
  return MOE_OK;
}

moe_status moe_ring_status(const moe_problem* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  int32_t* flag = nullptr;
  const moe_status st = moe_ring_error_flag(p, ws, ws_bytes, &flag);
  if (st != MOE_OK) return st;
  int32_t v = 0;
  (void)hipGetLastError();
  hipError_t e = hipMemcpyAsync(&v, flag, sizeof v, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return from_code(static_cast<int>(e));
  return v ? MOE_ERR_DEVICE : MOE_OK;
}

moe_status moe_forward_ring(const moe_problem* p, const void* x, const void* gate_w,
                            const float* bias, const void* W1t, const void* W3t, const void* W2t,
                            void* out, void* ws, size_t ws_bytes, const moe_debug* dbg,
                            hipStream_t stream) {
  return forward_impl(p, x, gate_w, bias, W1t, W3t, W2t, nullptr, nullptr, nullptr, out, ws,
                      ws_bytes, dbg, stream, true);
}

}  // extern "C"
