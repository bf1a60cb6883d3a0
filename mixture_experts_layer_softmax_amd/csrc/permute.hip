// permute.hip -- dispatch bookkeeping inside one GPU: expert histogram,
// exclusive scan, stable scatter of (token, k-slot) pairs to expert-ordered
// slots, and the expert tile map of the grouped GEMMs.
//
// The per-slot (token, k-slot) record is the one-device form of the source
// metadata every pool slot carries on the MegaMoE-vs-MoE-systems page
// (section 2.4); the layer stays dropless (section 2.6): every pair gets a
// slot and padding exists only in the tile map, never in memory (the local
// "in-place padding" idea of the FlashMoE Kernel page, Communication section).
//
// No atomics of any kind: each chunk of consecutive pairs is counted by one
// wavefront (ballot-matched lanes, one writer per expert) into a [chunks x E]
// table; one workgroup scans it in (expert,
// chunk) order; the scatter wavefront of each chunk re-ranks its pairs with
// ballots so equal experts keep increasing q = t*k + j order.  When all the
// pairs fit one chunk (decode), one workgroup does the three steps in a
// single launch.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// 64-bit mask of lanes in this wave holding the same value of `e` (bits 0..nb-1).
__device__ __forceinline__ uint64_t match_lanes(int e, int nbits, bool active) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    uint64_t ones = __ballot(active && ((e >> b) & 1));
    m &= ((e >> b) & 1) ? ones : ~ones;
  }
  return m;
}

// Count the experts of pairs [q0, q1) into cnt[] (LDS) with one wavefront and
// no atomics: in each group of 64 pairs, the lanes holding the same expert are
// found with ballots over the expert bits, and the last of them adds the
// group's count for that expert.  Distinct experts have distinct writers, and
// the groups run one after another, so every count is a plain add.
__device__ void count_run(const int32_t* __restrict__ ids, int q0, int q1, int nbits,
                          int32_t* cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int qb = q0; qb < q1; qb += 64) {
    const int q = qb + lane;
    const bool active = q < q1;
    const int e = active ? ids[q] : 0;
    const uint64_t peers = match_lanes(e, nbits, active);
    if (active && __popcll(peers & ~below) == 1) cnt[e] += __popcll(peers);  // last peer
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

__global__ __launch_bounds__(64) void hist_kernel(const int32_t* __restrict__ ids, int n,
                                                  int E, int nbits, int chunk,
                                                  int32_t* __restrict__ table) {
  extern __shared__ int32_t cnt[];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int q0 = blockIdx.x * chunk;
  count_run(ids, q0, min(n, q0 + chunk), nbits, cnt);
  __syncthreads();
  for (int e = lane; e < E; e += 64) table[static_cast<size_t>(blockIdx.x) * E + e] = cnt[e];
}

// Body of the scan for one workgroup of 1024 threads: tab [nchunk x E] (LDS
// or global) holds the per-(chunk, expert) counts and becomes, per cell, the
// slot base of that chunk inside its expert (without the expert's offset,
// which s_cnt[e] holds on return).  Also writes counts/offsets, the m-tile
// map for tile height bm and zeroes the GEMM work-queue counters.  The S
// shared experts (every token, after the routed slots) get their slot
// records and m-tiles here too.
__device__ void scan_core(int32_t* tab, int nchunk, int E, int bm, int32_t* __restrict__ counts,
                          int32_t* __restrict__ offsets, TileMap tm, int T, int k, int S,
                          int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_k,
                          int32_t* s_cnt) {
  __shared__ int32_t s_tiles[1024];
  __shared__ int32_t s_shared_tile0;  // first m-tile of the shared experts
  const int tid = threadIdx.x;
  int total = 0;
  if (tid < E) {
    // running sum down this expert's column; loads go out 8 at a time
    for (int c0 = 0; c0 < nchunk; c0 += 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = (c0 + u < nchunk) ? tab[static_cast<size_t>(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < nchunk) tab[static_cast<size_t>(c0 + u) * E + tid] = total;
        total += v[u];
      }
    }
  }
  const int tiles = (tid < E) ? (total + bm - 1) / bm : 0;
  s_cnt[tid] = (tid < E) ? total : 0;
  s_tiles[tid] = tiles;
  __syncthreads();
  // exclusive scans of counts and tiles over experts (E <= 1024); one
  // thread walks the experts in order -- at most 1024 steps
  if (tid == 0) {
    int acc_c = 0, acc_t = 0;
    for (int e = 0; e < E; ++e) {
      int c = s_cnt[e], t = s_tiles[e];
      s_cnt[e] = acc_c;
      s_tiles[e] = acc_t;
      acc_c += c;
      acc_t += t;
    }
    offsets[E] = acc_c;
    s_shared_tile0 = acc_t;
    *tm.n_mtiles = acc_t + S * ((T + bm - 1) / bm);
    for (int q = 0; q < kQueueWords; ++q) tm.queue[q] = 0;
  }
  __syncthreads();
  if (tid < E) {
    const int off = s_cnt[tid];
    counts[tid] = total;
    offsets[tid] = off;
    const int t0 = s_tiles[tid];
    for (int m = 0; m < tiles; ++m) {
      tm.e[t0 + m] = tid;
      tm.row0[t0 + m] = off + m * bm;
      tm.rows[t0 + m] = min(bm, total - m * bm);
    }
  }
  if (S > 0) {
    // shared experts: slot T*k + s*T + t holds (token t, k-slot k + s); their
    // m-tiles follow the routed ones, expert index E + s
    const int mt_per = (T + bm - 1) / bm, t_sh0 = s_shared_tile0;
    const int64_t base = static_cast<int64_t>(T) * k;
    for (int64_t i = tid; i < static_cast<int64_t>(S) * T; i += 1024) {
      slot_token[base + i] = static_cast<int32_t>(i % T);
      slot_k[base + i] = k + static_cast<int32_t>(i / T);
    }
    for (int i = tid; i < S * mt_per; i += 1024) {
      const int sh = i / mt_per, m = i - sh * mt_per;
      tm.e[t_sh0 + i] = E + sh;
      tm.row0[t_sh0 + i] = static_cast<int32_t>(base + static_cast<int64_t>(sh) * T + m * bm);
      tm.rows[t_sh0 + i] = min(bm, T - m * bm);
    }
  }
  __syncthreads();  // s_cnt (expert offsets) is final for the caller
}

// One workgroup of 1024 threads.  table [nchunk x E] in, becomes the base slot
// of each (chunk, expert); see scan_core for the rest.  When the table fits
// (LDS_TABLE), it is scanned in LDS: loaded and stored back coalesced by all
// threads, each expert's column summed by one thread from LDS.
template <bool LDS_TABLE>
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ table, int nchunk,
                                                    int E, int bm, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    TileMap tm, int T, int k, int S,
                                                    int32_t* __restrict__ slot_token,
                                                    int32_t* __restrict__ slot_k) {
  __shared__ int32_t s_cnt[1024];
  extern __shared__ int32_t s_tab[];  // [nchunk][E] when LDS_TABLE
  const int tid = threadIdx.x;
  const int cells = nchunk * E;
  if (LDS_TABLE) {
    for (int i = tid; i < cells; i += 1024) s_tab[i] = table[i];
    __syncthreads();
  }
  scan_core(LDS_TABLE ? s_tab : table, nchunk, E, bm, counts, offsets, tm, T, k, S, slot_token,
            slot_k, s_cnt);
  for (int i = tid; i < cells; i += 1024)
    table[i] = (LDS_TABLE ? s_tab[i] : table[i]) + s_cnt[i % E];
}

// Stable scatter of pairs [q0, q1) by one wavefront: base[e] is the next slot
// of expert e; ballots over the expert bits rank the lanes holding the same
// expert, so equal experts keep increasing q = t*k + j order.
__device__ void scatter_run(const int32_t* __restrict__ ids, int q0, int q1, int k, int nbits,
                            int32_t* base, int32_t* __restrict__ slot_token,
                            int32_t* __restrict__ slot_k, int32_t* __restrict__ token_slot) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int qb = q0; qb < q1; qb += 64) {
    const int q = qb + lane;
    const bool active = q < q1;
    const int e = active ? ids[q] : 0;
    const uint64_t peers = match_lanes(e, nbits, active);
    const int rank = __popcll(peers & below);
    const int cnt = __popcll(peers);
    int slot = 0;
    if (active) slot = base[e] + rank;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // every lane has read base[]
    if (active && rank == cnt - 1) base[e] += cnt;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (active) {
      slot_token[slot] = q / k;
      slot_k[slot] = q % k;
      token_slot[q] = slot;
    }
  }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                     int k, int E, int nbits, int chunk,
                                                     const int32_t* __restrict__ table,
                                                     int32_t* __restrict__ slot_token,
                                                     int32_t* __restrict__ slot_k,
                                                     int32_t* __restrict__ token_slot) {
  extern __shared__ int32_t base[];
  for (int e = threadIdx.x; e < E; e += 64)
    base[e] = table[static_cast<size_t>(blockIdx.x) * E + e];
  __syncthreads();
  const int q0 = blockIdx.x * chunk;
  scatter_run(ids, q0, min(n, q0 + chunk), k, nbits, base, slot_token, slot_k, token_slot);
}

// All of the permutation when the pairs fit one chunk (decode-sized T*k):
// histogram, scan and scatter in one workgroup, with the same results as the
// three kernels.
__global__ __launch_bounds__(1024) void permute_one_kernel(
    const int32_t* __restrict__ ids, int n, int E, int nbits, int bm, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, TileMap tm, int T, int k, int S,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_k,
    int32_t* __restrict__ token_slot) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_tab[1024];  // the one-chunk table: counts, then slot bases
  const int tid = threadIdx.x;
  if (tid < E) s_tab[tid] = 0;
  __syncthreads();
  if (tid < 64) count_run(ids, 0, n, nbits, s_tab);  // n <= one chunk of pairs
  __syncthreads();
  scan_core(s_tab, 1, E, bm, counts, offsets, tm, T, k, S, slot_token, slot_k, s_cnt);
  if (tid < E) s_tab[tid] += s_cnt[tid];
  __syncthreads();
  if (tid < 64) scatter_run(ids, 0, n, k, nbits, s_tab, slot_token, slot_k, token_slot);
}

__global__ __launch_bounds__(256) void zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) p[i] = 0;
}

}  // namespace

void launch_zero(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  zero_kernel<<<static_cast<int>(blocks), 256, 0, s>>>(p, n);
}

void launch_permute(const int32_t* ids, int T, int k, int E, int S, int bm, int32_t* table,
                    int32_t* counts, int32_t* offsets, int32_t* slot_token, int32_t* slot_k,
                    int32_t* token_slot, TileMap tm, hipStream_t s) {
  const int n = T * k;
  const int chunk = permute_chunk(n);
  const int nchunk = (n + chunk - 1) / chunk;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = sizeof(int32_t) * static_cast<size_t>(E);
  if (nchunk == 1) {
    permute_one_kernel<<<1, 1024, 0, s>>>(ids, n, E, nbits, bm, counts, offsets, tm, T, k, S,
                                          slot_token, slot_k, token_slot);
    return;
  }
  if (nchunk > 0) hist_kernel<<<nchunk, 64, lds, s>>>(ids, n, E, nbits, chunk, table);
  // the table in LDS when it fits next to the kernel's 8 KB of static LDS
  constexpr size_t kMaxTab = 144 * 1024;
  static const bool big_lds = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_kernel<true>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  static_cast<int>(kMaxTab)) == hipSuccess;
  const size_t tab_bytes = sizeof(int32_t) * static_cast<size_t>(nchunk) * E;
  if (tab_bytes <= (big_lds ? kMaxTab : 64 * 1024))
    scan_kernel<true><<<1, 1024, tab_bytes, s>>>(table, nchunk, E, bm, counts, offsets, tm, T,
                                                 k, S, slot_token, slot_k);
  else
    scan_kernel<false><<<1, 1024, 0, s>>>(table, nchunk, E, bm, counts, offsets, tm, T, k, S,
                                          slot_token, slot_k);
  if (nchunk > 0)
    scatter_kernel<<<nchunk, 64, lds, s>>>(ids, n, k, E, nbits, chunk, table, slot_token,
                                           slot_k, token_slot);
}

}  // namespace moe
