/*
 * moe.h -- C ABI of the MI355X MoE layer forward library (libmoe.so).
 *
 * One GPU runs a whole Mixture-of-Experts layer forward:
 *   softmax gate + top-k routing -> expert histogram and prefix-sum
 *   permutation -> grouped SwiGLU expert GEMMs -> gate-weighted combine.
 * The stage list is the one the FlashMoE Kernel page gives in its opening
 * paragraph (gate -> dispatch -> expert FFN -> combine), run here inside one
 * GPU with no exchange between devices.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises the host inside a call, except
 *    where an entry point says otherwise.
 *  - Every call enqueues its kernels on `stream` (NULL = the default stream)
 *    and returns immediately; outputs are valid once the caller synchronises
 *    the stream.
 *  - Arguments are checked before anything is enqueued.  On any error nothing
 *    is launched and no output is touched.  No C++ exception crosses the ABI.
 *  - Matrices are row-major and contiguous.  bf16 is IEEE bfloat16 storage
 *    (the upper half of an fp32); FP8 is OCP E4M3FN (max 448, no infinity).
 *  - No entry point reads a size back from the device, so a call can be
 *    captured into a HIP graph (the reason given on the FlashMoE Kernel page,
 *    "Problem" section, for why launch storms cannot simply be graphed is a
 *    host-sized pipeline; this one is device-sized).
 *  - Calls sharing one workspace must not overlap in time.
 *
 * Numerics (each choice is a reading where the pages are silent):
 *  - Router logits are fp32: acc = +0.0f, acc = fmaf(x[t][i], gate_w[i][e],
 *    acc) for i = 0 .. d-1 ascending, then acc + bias[e] as one fp32 add.
 *  - Top-k is taken on the logits; order is descending logit, equal logits
 *    ranked by lower expert index.  Weights are the softmax over the k
 *    selected logits (the renormalised full softmax), computed in fp64 and
 *    stored fp32.
 *  - Slots are ordered by expert, and inside an expert by q = t*k + j.
 *  - SwiGLU expert: h = SiLU(x W1) * (x W3), SiLU(a) = a / (1 + e^-a),
 *    y = h W2, fp32 accumulation; h is rounded to the activation format
 *    (fp32, bf16 RNE, FP8 1x128 groups, or MX FP8 blocks of 32 for
 *    MOE_MXFP4) before W2; y per slot stays fp32 (bf16 RNE on MXFP4 layers,
 *    whose 5e-2 tolerance absorbs that rounding).
 *  - FP8 groups: activations per 1x128 group along the contraction axis with
 *    scale s = amax / 448 (1 when amax == 0) and code e4m3_rne_sat(v / s)
 *    (both quotients fp32 IEEE); weights per 128x128 (K, N) block.
 *  - Combine: out[t] = sum_{j = 0 .. k-1} w[t][j] * y[slot(t, j)], fp32, in j
 *    order, then rounded (RNE) to out_dtype.  No floating-point atomics are
 *    used anywhere, so every output is bitwise reproducible run to run.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,          /* null pointer, bad size, bad dtype   */
    MOE_ERR_UNSUPPORTED = 2,          /* valid but not implemented shape     */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes < moe_workspace_size()     */
    MOE_ERR_HIP = 4,                  /* a HIP launch/runtime call failed    */
    MOE_ERR_DEVICE = 5                /* a bounded wait inside a launch gave
                                         up (reported by moe_ring_status)   */
} moe_status;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_FP8_E4M3 = 2,
    MOE_MXFP4 = 3   /* OCP MX FP4: E2M1 codes, E8M0 scale per 32 along K */
} moe_dtype;

/* Storage order of each expert's weight matrix (K = contraction length, N =
 * output columns: W1 and W3 are K = d by N = f, W2 is K = f by N = d).
 *   MOE_W_KN: row-major [K][N] per expert, the layout the workloads state
 *             (W1, W3 [E+S][d][f]; W2 [E+S][f][d]); FP8 codes the same, with
 *             [E+S][K/128][N/128] fp32 block scales.  moe_forward reads it as
 *             is for F32, BF16 and FP8 weights (the GEMMs stage k-rows of the
 *             weights in LDS and transpose them on the fragment read), with
 *             the same results bit for bit as MOE_W_NK; measured about 30 %
 *             slower per call than the packed layout on the bf16 prefill
 *             layer.  Not defined for MXFP4.
 *   MOE_W_NK: [N][K] per expert (contraction axis contiguous), the layout
 *             moe_pack_weight writes once, the faster one to read; MXFP4 codes
 *             [N][K/2] with their E8M0 scales packed by moe_pack_weight. */
typedef enum {
    MOE_W_KN = 0,
    MOE_W_NK = 1
} moe_weight_layout;

/* Problem description.  Sizes: T tokens, hidden d, expert intermediate f,
 * E experts, top_k experts per token (1 <= top_k <= E <= 1024).
 *   act_dtype: x and gate_w -- MOE_F32 or MOE_BF16.
 *   w_dtype:   W1, W3, W2   -- MOE_F32 (needs act_dtype F32), MOE_BF16 (needs
 *              act_dtype BF16), MOE_FP8_E4M3 (needs act_dtype BF16, d and f
 *              multiples of 128) or MOE_MXFP4 (needs act_dtype BF16, d and f
 *              multiples of 128): the FP8 x FP4 expert variant of the
 *              MegaMoE-vs-MoE-systems page (sections 1 and 4) in OCP MX form
 *              -- FP4 E2M1 weights with one E8M0 power-of-two scale per 32
 *              consecutive contraction elements, x and h quantised to MX FP8
 *              (E4M3, one E8M0 scale per 32) inside the layer, and the block
 *              scales applied by the scaled MFMA itself.
 *   out_dtype: MOE_F32 or MOE_BF16.
 *   block_m:   rows per expert tile of the grouped GEMMs; 0 picks it from the
 *              expected tokens per expert T*top_k/E (the serving-regime choice
 *              of the MegaMoE-vs-MoE-systems page, section 2.5, re-tuned for
 *              MFMA tiles).  Otherwise one of 16, 32, 64, 128, 256.
 * n_shared: shared experts, 0..8 (MegaMoE-vs-MoE-systems page, section 2.7:
 *            the shared expert's GEMMs are phases of the same task queue as
 *            the routed ones).  A shared expert sees every token and its
 *            output is added with weight 1 after the gate-weighted routed
 *            sum; its weights follow the E routed experts' in W1/W3/W2 (and
 *            their FP8 scales), which then hold E + n_shared experts.
 * w_layout: a moe_weight_layout, the storage order of W1, W3 and W2 (a
 *            zero-initialised problem means the stated [K][N] layout).
 * d and f must be multiples of 32 (fp32 weights), 64 (bf16) or 128 (FP8, MXFP4), and
 * x, h and one expert's weight matrix must each span less than 2^31 bytes
 * (MOE_ERR_UNSUPPORTED otherwise). */
typedef struct {
    int64_t T, d, f;
    int32_t E, top_k;
    int32_t act_dtype;
    int32_t w_dtype;
    int32_t out_dtype;
    int32_t block_m;
    int32_t n_shared;
    int32_t w_layout;
} moe_problem;

/* Optional device outputs filled from inside moe_forward, so that the routing
 * the fused call actually used can be compared with moe_route/moe_permute.
 * Any pointer may be NULL.  Sizes as in moe_route / moe_permute.
 * stage_events: caller-created HIP events (or NULL); event i is recorded on
 * the call's stream at stage boundary i: 0 start, 1 after the gate, 2 after
 * the FP8 / MX FP8 quantisation of x, 3 after histogram/scan/scatter, 4 after the
 * W1/W3 GEMM, 5 after the W2 GEMM, 6 after the combine.  Used to time each
 * kernel inside the whole-layer call.
 * gemm_clock: [2][2] uint64 device buffer, or NULL: for the W1/W3 (row 0) and
 * W2 (row 1) GEMM launches, the shader-clock ticks (s_memtime) and the
 * 100 MHz reference ticks (s_memrealtime) that the first workgroup spent from
 * its start to its exit -- the clock the chip sustained under that load is
 * 1e8 * ticks[0] / ticks[1] Hz. */
#define MOE_NUM_STAGE_EVENTS 7
typedef struct {
    int32_t *topk_ids;    /* [T*k]  */
    float *topk_w;        /* [T*k]  */
    int32_t *counts;      /* [E]    */
    int32_t *offsets;     /* [E+1]  */
    int32_t *slot_token;  /* [T*k]  */
    int32_t *slot_k;      /* [T*k]  */
    int32_t *token_slot;  /* [T*k]  */
    hipEvent_t stage_events[MOE_NUM_STAGE_EVENTS];
    uint64_t *gemm_clock; /* [2][2]: shader ticks, reference ticks per GEMM */
    /* moe_forward_ring only (moe_forward ignores both): polls, each a short
     * sleep, before a wait inside the launch gives up; 0 keeps the built-in
     * limit (seconds of polling); negative is MOE_ERR_INVALID_ARG. */
    int32_t ring_poll_limit;
    /* moe_forward_ring only, for testing the failure report: nonzero puts
     * every wait's target out of reach, so that each wait gives up after
     * ring_poll_limit polls (which must then be 1..4096, else
     * MOE_ERR_INVALID_ARG) and the error flag is set; the output is then
     * meaningless. */
    int32_t ring_force_timeout;
    /* moe_forward only: order in which each XCD's task queue hands out its
     * tasks -- 0 as laid out, 1 reversed, 2 a fixed shuffle (other values:
     * MOE_ERR_INVALID_ARG).  Every output element is written by one task, so
     * the output does not depend on it (the work-conserving queue of the
     * MegaMoE-vs-MoE-systems page, section 2.7, only decides who runs what). */
    int32_t queue_order;
    /* moe_forward only: NULL, or a device buffer of [2][task_log_capacity][4]
     * uint32 receiving one record per task of the W1/W3 (row 0) and W2 (row 1)
     * GEMM launches, at the task's index m_tile * n_tiles + n_tile: start time
     * and duration on the 100 MHz chip-wide reference clock (low 32 bits),
     * the workgroup that ran it, and 0x100 | the XCD it ran on.  Tasks with an
     * index >= task_log_capacity are not recorded; entries of tasks that do
     * not exist are left as they were. */
    uint32_t *task_log;
    int32_t task_log_capacity;
    /* moe_forward on FP8 and MXFP4 layers: NULL, or device buffers receiving
     * the activation codes and scales the expert GEMMs read, as the gate
     * wrote them: x_codes [T][d] E4M3 codes; x_scales FP8: [T][d/128] fp32,
     * MXFP4: [T][d/32] E8M0 bytes.  Ignored on other layers. */
    uint8_t *x_codes;
    void *x_scales;
    /* moe_forward only: NULL, or device buffers receiving the input rows of
     * the W2 GEMM (the SwiGLU output, rounded as W2 reads it) in slot order:
     * the T*k routed slots, then T rows per shared expert.
     *   h        [T*(k+n_shared)][f]  fp32 / bf16 layers: act_dtype values;
     *                                  FP8 and MXFP4 layers: E4M3 codes
     *   h_scales FP8: [T*(k+n_shared)][f/128] fp32; MXFP4: [..][f/32] E8M0
     *            bytes; ignored on other layers. */
    void *h;
    void *h_scales;
} moe_debug;

/* Human-readable name of a status code (static storage). */
const char *moe_status_string(moe_status s);

/* The HIP error code behind the last MOE_ERR_HIP on the calling thread. */
int moe_last_hip_error(void);

/* Bytes of device workspace that moe_route (when logits == NULL),
 * moe_permute and moe_forward need for this problem.  A pure function of the
 * problem, never of the routing: the dropless worst case of T*k slot rows
 * (the worst-case pool of the MegaMoE-vs-MoE-systems page, section 2.6, with
 * one rank) plus T rows per shared expert, tables, tile maps and FP8 scales. */
moe_status moe_workspace_size(const moe_problem *p, size_t *bytes);

/* Gate (FlashMoE Kernel page, opening paragraph: the first stage).
 *   x        [T][d]   act_dtype
 *   gate_w   [d][E]   act_dtype
 *   bias     [E]      fp32, or NULL (added to every logit of expert e)
 *   logits   [T][E]   fp32 output, or NULL (then kept in the workspace)
 *   topk_ids [T][k]   int32 output, descending logit, ties to lower index
 *   topk_w   [T][k]   fp32 output, renormalised softmax weights
 *   ws/ws_bytes       workspace; may be NULL/0 when logits != NULL.
 * d must be a multiple of 32 (MOE_ERR_UNSUPPORTED otherwise). */
moe_status moe_route(const moe_problem *p, const void *x, const void *gate_w,
                     const float *bias, float *logits, int32_t *topk_ids,
                     float *topk_w, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* Dispatch bookkeeping: atomic-free expert histogram, exclusive scan and
 * stable scatter (slot order by expert, then q = t*k + j).  The per-slot
 * source record (token, k-slot) is the one-GPU form of the source metadata
 * of the MegaMoE-vs-MoE-systems page, section 2.4.
 *   topk_ids   [T*k] int32 input, each in [0, E)  (out-of-range ids are
 *              undefined behaviour on the device; they are not detected)
 *   counts     [E]   rows per expert
 *   offsets    [E+1] exclusive scan of counts (offsets[E] == T*k)
 *   slot_token [T*k] source token of each slot
 *   slot_k     [T*k] source top-k index of each slot
 *   token_slot [T*k] inverse: slot of (t, j) at index t*k + j
 *   ws/ws_bytes workspace of at least moe_workspace_size().
 * Only the routed experts are permuted here (n_shared is ignored). */
moe_status moe_permute(const moe_problem *p, const int32_t *topk_ids,
                       int32_t *counts, int32_t *offsets, int32_t *slot_token,
                       int32_t *slot_k, int32_t *token_slot, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* FP8 1x128 group quantisation of a bf16 [rows][cols] matrix (cols % 128 ==
 * 0): q [rows][cols] E4M3FN codes, s [rows][cols/128] fp32 scales, as the FP8
 * layer applies it to x before the expert GEMMs. */
moe_status moe_quantize_fp8(int64_t rows, int64_t cols, const void *x_bf16,
                            uint8_t *q, float *s, hipStream_t stream);

/* OCP MX FP8 quantisation of a bf16 [rows][cols] matrix (cols % 32 == 0), as
 * the MXFP4 layer applies it to x: per block of 32 consecutive elements of a
 * row, X = floor(log2(amax)) - 8 (clamped to >= -127; 0 for an all-zero
 * block), s = X + 127 (E8M0 byte) and q = E4M3FN(v * 2^-X), round to nearest
 * even, saturating at 448.  q [rows][cols] codes, s [rows][cols/32] bytes. */
moe_status moe_quantize_mx(int64_t rows, int64_t cols, const void *x_bf16,
                           uint8_t *q, uint8_t *s, hipStream_t stream);

/* Bytes of each expert-weight tensor in the layout moe_forward reads
 * (element size of w_dtype times (E + n_shared)*d*f; MXFP4: half a byte per
 * element, the E8M0 scales, (E + n_shared)*d*f/32 bytes, not included). */
moe_status moe_weight_bytes(const moe_problem *p, size_t *bytes);

/* Optional one-time weight re-layout (untimed, done when weights are loaded): each
 * expert matrix given as [K][N] (W1, W3: [d][f]; W2: [f][d], the stated
 * layouts) is written as its transpose [N][K], so that the contraction axis
 * is contiguous for the MFMA operand loads.  src and dst must not overlap.
 * elem_bytes is 4 (fp32), 2 (bf16) or 1 (FP8 codes); E matrices of K x N.
 * MXFP4 weight codes are given already K-major and need no packing; their
 * E8M0 scales [E][N][K/32] are packed as E matrices of N x K/128 dwords.
 * MOE_ERR_UNSUPPORTED for K > 65535*64, N > 2^24 or E > 65535. */
moe_status moe_pack_weight(int32_t E, int64_t K, int64_t N, int32_t elem_bytes,
                           const void *src, void *dst, hipStream_t stream);

/* Whole layer forward: the operator the FlashMoE Kernel page describes in
 * its opening paragraph (gate -> dispatch -> expert FFN -> combine), for one
 * GPU and every token.  Routing is the renormalised top-k softmax gate of the
 * stated workloads; dispatch is dropless, each expert-ordered slot keeping
 * the (token, k-slot) it came from (MegaMoE-vs-MoE-systems page, sections 2.4
 * and 2.6); the expert FFN is SwiGLU; the combine is the gate-weighted sum
 * over each token's k slots (FlashMoE Kernel page, Architecture section).
 *   x       [T][d]       act_dtype
 *   gate_w  [d][E]       act_dtype
 *   bias    [E]          fp32 or NULL
 *   W1, W3  (gate, up) and W2 (down), E+S expert matrices each, in the order
 *           p->w_layout names:
 *             MOE_W_KN: W1, W3 [E+S][d][f], W2 [E+S][f][d] as stated;
 *             MOE_W_NK: W1, W3 [E+S][f][d], W2 [E+S][d][f], as written by
 *             moe_pack_weight (MXFP4: the same [N][K] shapes with two E2M1
 *             codes per byte, element 2i in the low nibble of byte i)
 *   W1s,W3s FP8: [E+S][d/128][f/128] fp32 block scales (either layout);
 *           MXFP4: E8M0 bytes, one per 32 elements along K, given as
 *           [E+S][f][d/32] and packed by moe_pack_weight (elem_bytes 4, the
 *           rows' dwords of 4 blocks transposed) to [E+S][d/128][f] dwords;
 *           NULL otherwise
 *   W2s     FP8: [E+S][f/128][d/128] fp32; MXFP4: [E+S][d][f/32] E8M0 bytes
 *           packed likewise to [E+S][f/128][d] dwords
 *           (S = n_shared: the shared experts follow the routed ones)
 *   out     [T][d]       out_dtype
 *   ws/ws_bytes          workspace of at least moe_workspace_size()
 *   dbg                  NULL, or device buffers receiving the routing used.
 * Kernels enqueued: route (logits, top-k; on FP8 and MXFP4 layers the same
 * pass over x writes its FP8 / MX FP8 codes and scales), histogram, scan +
 * tile map, scatter, grouped W1/W3 GEMM + SwiGLU, grouped W2 GEMM, combine.
 * Errors: MOE_ERR_INVALID_ARG (bad problem, NULL operand), MOE_ERR_UNSUPPORTED
 * (shape or layout the kernels do not cover, e.g. MOE_W_KN with MXFP4
 * weights, or FP8 weights with d or f above 32768), MOE_ERR_WORKSPACE_TOO_SMALL,
 * MOE_ERR_HIP (a launch failed; the
 * HIP code is kept for moe_last_hip_error).  All are returned before
 * anything is enqueued except MOE_ERR_HIP, after which the stream may hold
 * the kernels launched before the failing one. */
moe_status moe_forward(const moe_problem *p, const void *x, const void *gate_w,
                       const float *bias, const void *W1, const void *W3,
                       const void *W2, const void *W1s, const void *W3s,
                       const void *W2s, void *out, void *ws, size_t ws_bytes,
                       const moe_debug *dbg, hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc: moe_forward
 * with its workspace in a device array of the library itself
 * (MOE_NOALLOC_WORKSPACE_BYTES on each GPU it runs on, held until the process
 * ends).  Nothing is allocated inside the call, by the library or any routine
 * it calls; the caller still owns and passes every input and output, as in
 * moe_forward (same arguments, less ws/ws_bytes; same results bit for bit).
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give wrong results; the
 * array keeps the last call's contents, and every value a call reads from it
 * is written by the same call first.
 * MOE_ERR_WORKSPACE_TOO_SMALL (before anything is enqueued) when
 * moe_workspace_size(p) exceeds MOE_NOALLOC_WORKSPACE_BYTES -- a decode-sized
 * layer such as T = 64, d = 7168, f = 2048, E = 256, top_k = 8 needs 16 MB;
 * other errors as moe_forward. */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_problem *p, const void *x, const void *gate_w,
                               const float *bias, const void *W1, const void *W3,
                               const void *W2, const void *W1s, const void *W3s,
                               const void *W2s, void *out, const moe_debug *dbg,
                               hipStream_t stream);

/* The same layer forward with both expert GEMMs in ONE persistent launch
 * that hands h from the W1/W3 tasks to the W2 tasks through a bounded ring:
 * the ring of in-flight blocks (sized by blocks in flight, not by routed
 * tokens) and the L1/L2 full and empty counters of the MegaMoE-vs-MoE-systems
 * page, sections 2.3 and 2.7.  Each XCD's task queue runs, step by step, the
 * W1/W3 tasks of one work chunk and then the W2 tasks of the chunk two steps
 * back;
 * a W2 task waits until every W1/W3 task of its chunk has published its h
 * columns, and a W1/W3 task waits for its ring slot to be empty before
 * storing h.  h therefore needs 24 chunk-sized slots instead of T*k rows
 * (moe_ring_workspace_size); Y and everything else are as in moe_forward,
 * and the outputs are bit-identical to moe_forward's.
 * Supported: act_dtype = w_dtype = MOE_BF16, w_layout = MOE_W_NK, with
 * 256-row tiles (block_m 256, or block_m 0 when T*top_k/E picks 256);
 * otherwise MOE_ERR_UNSUPPORTED.
 * Arguments as in moe_forward (no weight scales); ws must hold
 * moe_ring_workspace_size() bytes.  The waits inside the launch are bounded:
 * a wait that exceeds its poll limit (seconds of polling by default; see
 * moe_debug) gives up, so the call cannot hang the device, but its output is
 * then wrong and moe_ring_error_flag's word reads 1. */
moe_status moe_ring_workspace_size(const moe_problem *p, size_t *bytes);
moe_status moe_forward_ring(const moe_problem *p, const void *x, const void *gate_w,
                            const float *bias, const void *W1t, const void *W3t,
                            const void *W2t, void *out, void *ws, size_t ws_bytes,
                            const moe_debug *dbg, hipStream_t stream);

/* Device address, inside ws, of the int32 error flag of moe_forward_ring:
 * every moe_forward_ring call on ws clears it to 0 before its GEMM launch,
 * and a wait inside that launch that gives up sets it to 1 (the call's
 * output is then wrong).  Read it on the call's stream once the call is done
 * (for instance hipMemcpyAsync to the host, then synchronise); the next call
 * on ws overwrites it.  No device work is enqueued here.
 * MOE_ERR_INVALID_ARG: p invalid, ws or flag NULL; MOE_ERR_UNSUPPORTED: as
 * moe_ring_workspace_size; MOE_ERR_WORKSPACE_TOO_SMALL: ws_bytes below
 * moe_ring_workspace_size(). */
moe_status moe_ring_error_flag(const moe_problem *p, void *ws, size_t ws_bytes,
                               int32_t **flag);

/* Outcome of the last moe_forward_ring call on ws: waits for `stream` (a host
 * synchronisation, unlike every other entry point), reads the error flag and
 * returns MOE_OK, or MOE_ERR_DEVICE when a bounded wait inside that launch
 * gave up (its output is then wrong).  Argument errors as
 * moe_ring_error_flag; MOE_ERR_HIP if the synchronisation or the read
 * fails. */
moe_status moe_ring_status(const moe_problem *p, void *ws, size_t ws_bytes,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
