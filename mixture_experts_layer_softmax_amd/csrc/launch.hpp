// launch.hpp -- host-side launch wrappers of the HIP kernels and the small
// structs they share with api.cpp.  Internal to libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// (token, k) pairs per histogram/scatter chunk: enough chunks to spread the
// scatter over many wavefronts, few enough for the single-workgroup scan.
constexpr int kPermuteMinChunk = 512;
constexpr int kPermuteMaxChunks = 128;
inline int permute_chunk(long long n) {
  long long c = (n + kPermuteMaxChunks - 1) / kPermuteMaxChunks;
  c = (c + 63) / 64 * 64;
  return static_cast<int>(c < kPermuteMinChunk ? kPermuteMinChunk : c);
}

constexpr int kQueueWords = 16;  // 8 per-XCD work-queue counters per GEMM

// Largest number of 128-element contraction blocks of an FP8 GEMM (the
// kernel stages a tile's weight block scales in LDS): d, f <= 32768.
constexpr int kWscMax = 256;

// Expert m-tile map written by the scan kernel: tile i covers slots
// [row0[i], row0[i] + rows[i]) of expert e[i].  n_mtiles is the number of
// valid entries; queue[kQueueWords] are the per-XCD work-queue counters of
// the two GEMMs (zeroed by the scan kernel).
struct TileMap {
  int32_t* e;
  int32_t* row0;
  int32_t* rows;
  int32_t* n_mtiles;
  int32_t* queue;
};

// dtype codes (same values as moe_dtype); kMX4 = FP4 (E2M1) weights with
// E8M0 block scales, the activations MX FP8
constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2, kMX4 = 3;

struct GemmArgs {
  // activation operand: rows of K elements
  const uint8_t* A;
  int64_t a_row_bytes;
  int64_t a_bytes;        // bytes of the buffer A points into (its rows' extent)
  const int32_t* gather;  // row index table (slot -> token), or null (row = slot)
  const float* sa;        // FP8: [rows][sa_stride] scales of A rows (K/128 used); MX: E8M0
                          // bytes [rows][K/32]
  int sa_stride;          // FP8: floats per A-row scale row, a multiple of 4
  int64_t sa_bytes;       // FP8: bytes of the buffer sa points into
  // weight operand(s): [E][N][K] (contraction axis contiguous)
  const uint8_t* B0;      // W1t (phase 1) or W2t (phase 2)
  const uint8_t* B1;      // W3t (phase 1)
  const float* sb0;       // FP8: [E][K/128][N/128]; MX: E8M0 bytes [E][N][K/32]
  const float* sb1;
  int64_t K;              // contraction length (elements)
  int64_t N;              // output columns: f (phase 1) or d (phase 2)
  // outputs
  uint8_t* C;             // h [slots][f] (phase 1) or Y [slots][d] (phase 2: fp32 for fp32
                          // layers, bf16 for MXFP4, else fp16 codes under the scales in ce)
  uint8_t* ce;            // phase 2, fp16 Y: exponent byte x + 127 per 32 columns
                          // [slots][d/32]; Y = code * 2^x
  float* sc;              // phase 1 h scales: FP8 [slots][sc_stride]; MX E8M0 bytes [slots][f/32]
  int sc_stride;          // FP8: floats per h scale row, a multiple of 4
  TileMap tm;
  int n_tiles_n;          // column tiles per m-tile
  int queue_idx;
  int group_m;            // m-tiles per XCD work chunk (1..8)
  int stream_c;           // phase 2: store Y with non-temporal hints (Y far beyond the MALL)
  uint64_t* clock;        // [2] or null: ticks of workgroup 0 (shader, 100 MHz reference)
  int queue_order;        // debug: 0 as laid out, 1 reversed, 2 shuffled task order
  uint32_t* task_log;     // debug: [task_log_capacity][4] per-task records, or null
  int task_log_capacity;
};

// Single-launch W1/W3 -> W2 pipeline (bf16, 256 x 256 tiles) through a
// bounded ring of h.  XCD y's queue runs steps s = 0, 1, ..: the W1/W3 tasks
// of its chunk s, then the W2 tasks of its chunk s - kRingLag.  Chunk j of
// XCD y writes its h into ring slot y * slots + j % slots (group_m * 256
// rows), once the W2 tasks of chunk j - slots (step j - slots + kRingLag) are
// done.  Every wait then targets tasks earlier in the same queue as long as
// slots > kRingLag.  All counters are zeroed before the launch.
// Two steps between a chunk's W1/W3 and W2 tasks leave its W1/W3 tasks time
// to finish before its W2 tasks are pulled (measured against one step:
// 2 % shorter on prefill, 5 % on the skewed layer).
constexpr int kRingLag = 2;
struct RingArgs {
  uint8_t* h;        // [8 * slots][group_m * 256 rows][f] bf16
  int32_t* queue;    // [8] pull counters
  int32_t* l1_done;  // [chunks] finished W1/W3 tasks per chunk (full count)
  int32_t* l2_done;  // [chunks] finished W2 tasks per chunk (empty count)
  int32_t* err;      // [1] set to 1 when a bounded wait gave up
  int slots;         // ring slots per XCD (> kRingLag)
  int poll_limit;    // polls (each a short sleep) before a wait gives up
  int unreachable;   // 0, or 1 << 30 to put every wait's target out of reach
};
// Default poll limit of the ring waits: seconds of polling, far beyond any
// wait of a healthy launch.
constexpr int kRingPollLimit = 1 << 22;
// Largest poll limit a caller may set together with unreachable targets.
constexpr int kRingForcedPollMax = 4096;

// Gate: logits [T][E] (+ bias), top-k ids and renormalised weights [T][k].
// quant 1 / 2 also writes x (bf16) quantised to FP8 1x128 groups (codes xq
// [T][d], fp32 scales xs [T][xs_stride]) or to MX FP8 blocks of 32 (codes xq,
// E8M0 bytes xs [T][d/32]) in the same pass.  Returns a hipError_t.
int launch_gate(const void* x, const void* gate_w, const float* bias, float* logits,
                int32_t* ids, float* w, int T, int d, int E, int k, bool bf16, hipStream_t s,
                int quant = 0, uint8_t* xq = nullptr, void* xs = nullptr, int64_t xs_stride = 0);
// S shared experts add T slots each after the T*k routed ones (slot
// T*k + s*T + t holds token t, k-slot k + s) and their m-tiles after the
// routed ones.
void launch_permute(const int32_t* ids, int T, int k, int E, int S, int bm, int32_t* table,
                    int32_t* counts, int32_t* offsets, int32_t* slot_token, int32_t* slot_k,
                    int32_t* token_slot, TileMap tm, hipStream_t s);
// s has s_stride floats per row (cols/128 of them written).
void launch_quant_fp8(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* s,
                      int64_t s_stride, hipStream_t st);
// MX FP8: blocks of 32 along the row, E4M3 codes + E8M0 scale bytes [rows][cols/32].
void launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                     hipStream_t st);
// Grouped GEMMs.  bm = tile height; wkn: weights in the stated [E][K][N]
// layout (else the packed [E][N][K]); returns a hipError_t (-1: no kernel
// for this combination).
int launch_gemm(int phase, int dtype, int bm, bool wkn, const GemmArgs& a, hipStream_t s);
// Both GEMMs in one launch through the h ring (bf16 weights, bm = 256); g1.C
// and g2.A point at r.h.  Returns a hipError_t.
int launch_gemm_ring(const GemmArgs& g1, const GemmArgs& g2, const RingArgs& r, hipStream_t s);
// Zero n int32 words with a kernel (also inside a captured graph).
void launch_zero(int32_t* p, int64_t n, hipStream_t s);
// Column tiles per m-tile for a phase (depends on the kernel variant).
int gemm_tile_n(int phase, int dtype, int bm, bool wkn);
// Formats of Y [T*k + S*T][d]: fp32, bf16, or fp16 codes with one exponent
// byte x + 127 per 32 columns in ye [T*k + S*T][d/32] (Y = code * 2^x).
enum YFormat { kYF32 = 0, kYBF16 = 1, kYF16E = 2 };
void launch_combine(const void* Y, int y_format, const uint8_t* ye, const float* w,
                    const int32_t* token_slot, void* out, int T, int d, int k, int S,
                    bool out_bf16, hipStream_t s);
void launch_pack(int E, int64_t K, int64_t N, int elem_bytes, const void* src, void* dst,
                 hipStream_t s);

}  // namespace moe
