"""ctypes binding of libmoe.so -- argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI of include/moe.h, and
raises on a non-OK status.  Nothing here computes any part of the layer; if
libmoe.so is missing the import fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
MOE_W_KN, MOE_W_NK = 0, 1  # weight storage order: as stated [K][N], or packed [N][K]
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP", 5: "MOE_ERR_DEVICE"}

EXPORTS = ["moe_status_string", "moe_last_hip_error", "moe_workspace_size", "moe_route",
           "moe_permute", "moe_quantize_fp8", "moe_quantize_mx", "moe_weight_bytes",
           "moe_pack_weight", "moe_forward", "moe_ring_workspace_size", "moe_forward_ring",
           "moe_ring_error_flag", "moe_ring_status", "moe_forward_noalloc"]
NOALLOC_WORKSPACE_BYTES = 64 << 20  # MOE_NOALLOC_WORKSPACE_BYTES


class MoEProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64),
                ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("w_layout", ctypes.c_int32)]


NUM_STAGE_EVENTS = 7
DEBUG_BUFFERS = ("topk_ids", "topk_w", "counts", "offsets", "slot_token", "slot_k",
                 "token_slot")


class MoEDebug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in DEBUG_BUFFERS] + [
        ("stage_events", ctypes.c_void_p * NUM_STAGE_EVENTS),
        ("gemm_clock", ctypes.c_void_p),
        ("ring_poll_limit", ctypes.c_int32), ("ring_force_timeout", ctypes.c_int32),
        ("queue_order", ctypes.c_int32), ("task_log", ctypes.c_void_p),
        ("task_log_capacity", ctypes.c_int32), ("x_codes", ctypes.c_void_p),
        ("x_scales", ctypes.c_void_p), ("h", ctypes.c_void_p), ("h_scales", ctypes.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, fn, code, hip):
        self.code = code
        self.hip = hip
        super().__init__(f"{fn} -> {STATUS.get(code, code)}"
                         + (f" (hip error {hip})" if code == 4 else ""))


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (built in-tree by build()); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run __graft_entry__.build() or "
                          "python -m mixture_experts_layer_softmax_amd.build")
    lib = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    PP = ctypes.POINTER(MoEProblem)
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_hip_error.restype = ctypes.c_int
    lib.moe_workspace_size.argtypes = [PP, ctypes.POINTER(S)]
    lib.moe_weight_bytes.argtypes = [PP, ctypes.POINTER(S)]
    lib.moe_route.argtypes = [PP, P, P, P, P, P, P, P, S, P]
    lib.moe_permute.argtypes = [PP, P, P, P, P, P, P, P, S, P]
    lib.moe_quantize_fp8.argtypes = [ctypes.c_int64, ctypes.c_int64, P, P, P, P]
    lib.moe_quantize_mx.argtypes = [ctypes.c_int64, ctypes.c_int64, P, P, P, P]
    lib.moe_pack_weight.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, P, P, P]
    lib.moe_forward.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, S,
                                ctypes.POINTER(MoEDebug), P]
    lib.moe_ring_workspace_size.argtypes = [PP, ctypes.POINTER(S)]
    lib.moe_forward_ring.argtypes = [PP, P, P, P, P, P, P, P, P, S, ctypes.POINTER(MoEDebug), P]
    lib.moe_ring_error_flag.argtypes = [PP, P, S, ctypes.POINTER(P)]
    lib.moe_ring_status.argtypes = [PP, P, S, P]
    lib.moe_forward_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P,
                                        ctypes.POINTER(MoEDebug), P]
    for fn in EXPORTS:
        if fn not in ("moe_status_string", "moe_last_hip_error"):
            getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise MoEError(fn, rc, load().moe_last_hip_error())


def problem(T, d, f, E, top_k, act_dtype, w_dtype, out_dtype, block_m=0,
            n_shared=0, w_layout=MOE_W_NK) -> MoEProblem:
    """moe_problem; w_layout defaults to the packed [N][K] weights that
    pack_weights() produces."""
    return MoEProblem(T, d, f, E, top_k, act_dtype, w_dtype, out_dtype, block_m, n_shared,
                      w_layout)


def problem_of(cfg, T=None, block_m=0, out_dtype=None, w_layout=MOE_W_NK) -> MoEProblem:
    return problem(cfg.T if T is None else T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.act_dtype,
                   cfg.w_dtype, cfg.out_dtype if out_dtype is None else out_dtype, block_m,
                   cfg.n_shared, w_layout)


def workspace_size(p: MoEProblem) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", load().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def weight_bytes(p: MoEProblem) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_weight_bytes", load().moe_weight_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def alloc_workspace(p: MoEProblem, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_size(p), dtype=torch.uint8, device=device)


def ring_workspace_size(p: MoEProblem) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_ring_workspace_size",
           load().moe_ring_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_route(p, x, gate_w, bias, logits, topk_ids, topk_w, ws=None, stream=None):
    rc = load().moe_route(ctypes.byref(p), _p(x), _p(gate_w), _p(bias), _p(logits),
                          _p(topk_ids), _p(topk_w), _p(ws),
                          0 if ws is None else ws.numel(), _stream(stream))
    _check("moe_route", rc)


def moe_permute(p, topk_ids, counts, offsets, slot_token, slot_k, token_slot, ws,
                stream=None):
    rc = load().moe_permute(ctypes.byref(p), _p(topk_ids), _p(counts), _p(offsets),
                            _p(slot_token), _p(slot_k), _p(token_slot), _p(ws), ws.numel(),
                            _stream(stream))
    _check("moe_permute", rc)


def moe_quantize_fp8(x_bf16, q, s, stream=None):
    rows, cols = x_bf16.shape
    rc = load().moe_quantize_fp8(rows, cols, _p(x_bf16), _p(q), _p(s), _stream(stream))
    _check("moe_quantize_fp8", rc)


def moe_quantize_mx(x_bf16, q, s, stream=None):
    rows, cols = x_bf16.shape
    rc = load().moe_quantize_mx(rows, cols, _p(x_bf16), _p(q), _p(s), _stream(stream))
    _check("moe_quantize_mx", rc)


def moe_pack_weight(src, dst, stream=None):
    """src [E][K][N] -> dst [E][N][K] (any 1/2/4-byte element type)."""
    E, K, N = src.shape
    rc = load().moe_pack_weight(E, K, N, src.element_size(), _p(src), _p(dst),
                                _stream(stream))
    _check("moe_pack_weight", rc)


def moe_forward(p, x, gate_w, bias, W1, W3, W2, W1s, W3s, W2s, out, ws, dbg=None,
                stream=None):
    dbg_s = _debug_struct(dbg)
    rc = load().moe_forward(ctypes.byref(p), _p(x), _p(gate_w), _p(bias), _p(W1), _p(W3),
                            _p(W2), _p(W1s), _p(W3s), _p(W2s), _p(out), _p(ws), ws.numel(),
                            None if dbg_s is None else ctypes.byref(dbg_s), _stream(stream))
    _check("moe_forward", rc)


def moe_forward_noalloc(p, x, gate_w, bias, W1, W3, W2, W1s, W3s, W2s, out, dbg=None,
                        stream=None):
    """moe_forward with the library's own static workspace (no allocation)."""
    dbg_s = _debug_struct(dbg)
    rc = load().moe_forward_noalloc(ctypes.byref(p), _p(x), _p(gate_w), _p(bias), _p(W1),
                                    _p(W3), _p(W2), _p(W1s), _p(W3s), _p(W2s), _p(out),
                                    None if dbg_s is None else ctypes.byref(dbg_s),
                                    _stream(stream))
    _check("moe_forward_noalloc", rc)


def _debug_struct(dbg):
    if dbg is None:
        return None
    dbg_s = MoEDebug(*[None if dbg.get(n) is None else dbg[n].data_ptr() for n in DEBUG_BUFFERS])
    for i, ev in enumerate(dbg.get("stage_events") or []):
        dbg_s.stage_events[i] = ev
    if dbg.get("gemm_clock") is not None:
        dbg_s.gemm_clock = dbg["gemm_clock"].data_ptr()
    dbg_s.ring_poll_limit = int(dbg.get("ring_poll_limit", 0))
    dbg_s.ring_force_timeout = int(dbg.get("ring_force_timeout", 0))
    dbg_s.queue_order = int(dbg.get("queue_order", 0))
    for name in ("x_codes", "x_scales", "h", "h_scales"):
        if dbg.get(name) is not None:
            setattr(dbg_s, name, dbg[name].data_ptr())
    if dbg.get("task_log") is not None:  # uint32 tensor [2][capacity][4]
        dbg_s.task_log = dbg["task_log"].data_ptr()
        dbg_s.task_log_capacity = int(dbg["task_log"].shape[1])
    return dbg_s


def moe_forward_ring(p, x, gate_w, bias, W1t, W3t, W2t, out, ws, dbg=None, stream=None):
    dbg_s = _debug_struct(dbg)
    rc = load().moe_forward_ring(ctypes.byref(p), _p(x), _p(gate_w), _p(bias), _p(W1t),
                                 _p(W3t), _p(W2t), _p(out), _p(ws), ws.numel(),
                                 None if dbg_s is None else ctypes.byref(dbg_s), _stream(stream))
    _check("moe_forward_ring", rc)


def moe_ring_error_flag(p, ws):
    """Device address of the ring error flag inside the workspace tensor ws."""
    addr = ctypes.c_void_p()
    rc = load().moe_ring_error_flag(ctypes.byref(p), _p(ws), ws.numel(), ctypes.byref(addr))
    _check("moe_ring_error_flag", rc)
    return addr.value


def moe_ring_status(p, ws, stream=None) -> int:
    """Status of the last moe_forward_ring call on ws (waits for the stream):
    0 (MOE_OK) or 5 (MOE_ERR_DEVICE, a wait inside the launch gave up)."""
    rc = load().moe_ring_status(ctypes.byref(p), _p(ws), ws.numel(), _stream(stream))
    if rc not in (0, 5):
        _check("moe_ring_status", rc)
    return rc


def ring_failed(p, ws, stream=None):
    """True when a wait of the last moe_forward_ring call on ws gave up
    (moe_ring_status returned MOE_ERR_DEVICE)."""
    return moe_ring_status(p, ws, stream) == 5


# ---------------------------------------------------------------------------
# convenience wrappers over the calls above (tensor allocation + marshalling)
# ---------------------------------------------------------------------------

def pack_weights(inp: dict, stream=None) -> dict:
    """One-time re-layout of W1/W3/W2 ([E][K][N] -> [E][N][K]) on the GPU.
    MXFP4 weights (uint8 E8M0 scales) come K-major already; their scales
    [E][N][K/32] are re-laid as [E][K/128][N] dwords (4 blocks of 32 each)."""
    out = {}
    if inp.get("W1s") is not None and inp["W1s"].dtype == torch.uint8:
        out = {"W1t": inp["W1"], "W3t": inp["W3"], "W2t": inp["W2"]}
        for name in ("W1s", "W3s", "W2s"):
            sc = inp[name]
            E, N, KB = sc.shape
            src = sc.view(torch.int32)  # [E][N][K/128] dwords
            dst = torch.empty((E, KB // 4, N), dtype=torch.int32, device=sc.device)
            moe_pack_weight(src, dst, stream)
            out[name] = dst.view(torch.uint8)
        return out
    for name in ("W1", "W3", "W2"):
        w = inp[name]
        E, K, N = w.shape
        dst = torch.empty((E, N, K), dtype=w.dtype, device=w.device)
        moe_pack_weight(w, dst, stream)
        out[name + "t"] = dst
    for name in ("W1s", "W3s", "W2s"):
        out[name] = inp.get(name)
    return out


def out_tensor(cfg, T=None, device="cuda", out_dtype=None):
    od = cfg.out_dtype if out_dtype is None else out_dtype
    return torch.empty((cfg.T if T is None else T, cfg.d),
                       dtype=torch.float32 if od == MOE_F32 else torch.bfloat16, device=device)


def forward(cfg, inp: dict, packed: dict | None, out=None, ws=None, dbg=None, out_dtype=None,
            block_m=0, stream=None, ring=False):
    """Whole-layer forward of cfg on resident inputs; returns the output tensor.
    packed: weights from pack_weights() (layout MOE_W_NK), or None to pass
    inp's weights in the stated [K][N] layout (MOE_W_KN).
    ring=True runs moe_forward_ring (both GEMMs in one launch, h in a ring)."""
    T = inp["x"].shape[0]
    layout = MOE_W_KN if packed is None else MOE_W_NK
    p = problem_of(cfg, T=T, block_m=block_m, out_dtype=out_dtype, w_layout=layout)
    if packed is None:
        W1, W3, W2 = inp["W1"], inp["W3"], inp["W2"]
        W1s, W3s, W2s = inp.get("W1s"), inp.get("W3s"), inp.get("W2s")
    else:
        W1, W3, W2 = packed["W1t"], packed["W3t"], packed["W2t"]
        W1s, W3s, W2s = packed.get("W1s"), packed.get("W3s"), packed.get("W2s")
    if out is None:
        out = out_tensor(cfg, T=T, device=inp["x"].device, out_dtype=out_dtype)
    if ws is None:
        size = ring_workspace_size(p) if ring else workspace_size(p)
        ws = torch.empty(size, dtype=torch.uint8, device=inp["x"].device)
    if ring:
        moe_forward_ring(p, inp["x"], inp["gate_w"], inp.get("bias"), W1, W3, W2, out, ws,
                         dbg=dbg, stream=stream)
    else:
        moe_forward(p, inp["x"], inp["gate_w"], inp.get("bias"), W1, W3, W2, W1s, W3s, W2s,
                    out, ws, dbg=dbg, stream=stream)
    return out
