"""ctypes binding of liboracle.so (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Arrays are numpy arrays in host memory.  bf16 data is passed as its raw
``uint16`` bit patterns, FP8 E4M3FN data as ``uint8`` codes, MX FP4 (E2M1)
data as one ``uint8`` code per element and MX scales as ``uint8`` E8M0 bytes,
so the oracle reads exactly the bits the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

ORC_F32, ORC_BF16, ORC_FP8, ORC_MXFP4 = 0, 1, 2, 3
MX_E4M3, MX_E2M1 = 0, 1  # element formats of MX blocks

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("f", ctypes.c_int64),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
    ]


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (plain gcc + OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_route.argtypes = [ctypes.POINTER(_Problem), P, P, P, P, P, P]
    lib.orc_route.restype = ctypes.c_int
    lib.orc_permute.argtypes = [i64, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P]
    lib.orc_permute.restype = ctypes.c_int
    lib.orc_forward.argtypes = [ctypes.POINTER(_Problem), P, P, P, P, P, P, P, P, P,
                                P, i64, P, P, P]
    lib.orc_forward.restype = ctypes.c_int
    lib.orc_expert_hidden.argtypes = [ctypes.POINTER(_Problem), P, i64, P, P, P, P, P]
    lib.orc_expert_hidden.restype = ctypes.c_int
    lib.orc_fp8_quant_rows.argtypes = [i64, i64, P, P, P]
    lib.orc_e4m3_encode_array.argtypes = [i64, P, P]
    lib.orc_e4m3_decode_array.argtypes = [i64, P, P]
    lib.orc_round_bf16_array.argtypes = [i64, P, P]
    lib.orc_e2m1_encode_array.argtypes = [i64, P, P]
    lib.orc_e2m1_decode_array.argtypes = [i64, P, P]
    lib.orc_mx_exponent.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.orc_mx_exponent.restype = ctypes.c_int
    lib.orc_mx_quant_rows.argtypes = [i64, i64, ctypes.c_int, P, P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _act(a, act_dtype):
    return _c(a, np.float32 if act_dtype == ORC_F32 else np.uint16)


def _problem(T, d, f, E, k, act_dtype, w_dtype, n_shared=0):
    return _Problem(T, d, f, E, k, act_dtype, w_dtype, n_shared)


def route(x, gate_w, bias, k, act_dtype):
    """Gate of every token.  x [T x d], gate_w [d x E] (fp32, or bf16 bits as
    uint16), bias [E] fp32 or None.  Returns (logits fp32 [T x E],
    ids int32 [T x k], w fp32 [T x k])."""
    lib = _load()
    x = _act(x, act_dtype)
    gate_w = _act(gate_w, act_dtype)
    T, d = x.shape
    E = gate_w.shape[1]
    bias = None if bias is None else _c(bias, np.float32)
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    p = _problem(T, d, 0, E, k, act_dtype, act_dtype)
    rc = lib.orc_route(ctypes.byref(p), _ptr(x), _ptr(gate_w), _ptr(bias),
                       _ptr(logits), _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("orc_route rejected its arguments")
    return logits, ids, w


def permute(ids, E):
    """Histogram, exclusive scan and stable scatter of ids [T x k].
    Returns dict of counts [E], offsets [E+1], slot_token, slot_k, token_slot
    (each [T*k], int32)."""
    lib = _load()
    ids = _c(ids, np.int32)
    T, k = ids.shape
    n = T * k
    out = {
        "counts": np.empty(E, np.int32),
        "offsets": np.empty(E + 1, np.int32),
        "slot_token": np.empty(n, np.int32),
        "slot_k": np.empty(n, np.int32),
        "token_slot": np.empty(n, np.int32),
    }
    rc = lib.orc_permute(T, k, E, _ptr(ids), _ptr(out["counts"]), _ptr(out["offsets"]),
                         _ptr(out["slot_token"]), _ptr(out["slot_k"]), _ptr(out["token_slot"]))
    if rc:
        raise ValueError("orc_permute: expert id out of range")
    return out


def forward(x, gate_w, bias, W1, W3, W2, k, act_dtype, w_dtype, tokens=None,
            W1s=None, W3s=None, W2s=None, n_shared=0):
    """Layer forward for the listed tokens (all tokens if None).

    W1, W3, W2: sequences of E + n_shared per-expert arrays ([d x f],
    [d x f], [f x d]), the n_shared shared experts last; a routed entry may
    be None for an expert none of the listed tokens routes to.  Shared
    experts see every token and are added with weight 1.
    For FP8 weights (uint8 codes) W1s/W3s/W2s hold each expert's fp32
    [K/128 x N/128] block scales; for MXFP4 weights (one uint8 E2M1 code per
    element) they hold each expert's [K/32 x N] uint8 E8M0 scales.
    Returns (out fp64 [ntok x d] unrounded, ids [ntok x k], w [ntok x k]).
    """
    lib = _load()
    x = _act(x, act_dtype)
    gate_w = _act(gate_w, act_dtype)
    T, d = x.shape
    E = gate_w.shape[1]
    f = None
    wdt = {ORC_F32: np.float32, ORC_BF16: np.uint16, ORC_FP8: np.uint8,
           ORC_MXFP4: np.uint8}[w_dtype]
    keep = []

    ne = E + n_shared

    def plist(arrs, dt):
        ptrs = (ctypes.c_void_p * ne)()
        for e in range(ne):
            a = None if arrs is None else arrs[e]
            if a is not None:
                a = _c(a, dt)
                keep.append(a)
                ptrs[e] = a.ctypes.data
        return ptrs

    for a in W1:
        if a is not None:
            f = a.shape[1]
            break
    if f is None:
        raise ValueError("no expert weights given")
    p1, p3, p2 = plist(W1, wdt), plist(W3, wdt), plist(W2, wdt)
    sdt = {ORC_FP8: np.float32, ORC_MXFP4: np.uint8}.get(w_dtype)
    s1 = plist(W1s, sdt) if sdt else None
    s3 = plist(W3s, sdt) if sdt else None
    s2 = plist(W2s, sdt) if sdt else None
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = _c(np.asarray(tokens, dtype=np.int64), np.int64)
    ntok = tokens.shape[0]
    bias = None if bias is None else _c(bias, np.float32)
    out = np.empty((ntok, d), np.float64)
    ids = np.empty((ntok, k), np.int32)
    w = np.empty((ntok, k), np.float32)
    p = _problem(T, d, f, E, k, act_dtype, w_dtype, n_shared)
    cp = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    rc = lib.orc_forward(ctypes.byref(p), _ptr(x), _ptr(gate_w), _ptr(bias),
                         cp(p1), cp(p3), cp(p2), cp(s1), cp(s3), cp(s2),
                         _ptr(tokens), ntok, _ptr(out), _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("orc_forward rejected its arguments (bad token or missing expert)")
    return out, ids, w


def expert_hidden(x, t, W1, W3, act_dtype, w_dtype, W1s=None, W3s=None):
    """Exact SwiGLU output of token t through one expert, before it is
    rounded to the format W2 reads: fp64 [f].  x is the full [T x d]
    activation matrix (fp32, or bf16 bits as uint16); W1, W3 one expert's
    [d x f] weights in the layout forward() takes, W1s/W3s their scales for
    FP8 and MXFP4 weights."""
    lib = _load()
    x = _act(x, act_dtype)
    T, d = x.shape
    wdt = {ORC_F32: np.float32, ORC_BF16: np.uint16, ORC_FP8: np.uint8,
           ORC_MXFP4: np.uint8}[w_dtype]
    W1, W3 = _c(W1, wdt), _c(W3, wdt)
    f = W1.shape[1]
    sdt = {ORC_FP8: np.float32, ORC_MXFP4: np.uint8}.get(w_dtype)
    if sdt is not None:
        W1s, W3s = _c(W1s, sdt), _c(W3s, sdt)
    else:
        W1s = W3s = None
    h = np.empty(f, np.float64)
    p = _problem(T, d, f, 1, 1, act_dtype, w_dtype)
    if lib.orc_expert_hidden(ctypes.byref(p), _ptr(x), int(t), _ptr(W1), _ptr(W3),
                             _ptr(W1s), _ptr(W3s), _ptr(h)):
        raise ValueError("orc_expert_hidden: token out of range")
    return h


def fp8_quant_rows(v):
    """1x128 group quantisation of an fp32 [rows x cols] matrix.
    Returns (codes uint8 [rows x cols], scales fp32 [rows x ceil(cols/128)])."""
    lib = _load()
    v = _c(v, np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, (cols + 127) // 128), np.float32)
    lib.orc_fp8_quant_rows(rows, cols, _ptr(v), _ptr(q), _ptr(s))
    return q, s


def e4m3_encode(v):
    lib = _load()
    v = _c(np.asarray(v, np.float32).ravel(), np.float32)
    q = np.empty(v.shape, np.uint8)
    lib.orc_e4m3_encode_array(v.size, _ptr(v), _ptr(q))
    return q


def e4m3_decode(q):
    lib = _load()
    q = _c(np.asarray(q, np.uint8).ravel(), np.uint8)
    v = np.empty(q.shape, np.float64)
    lib.orc_e4m3_decode_array(q.size, _ptr(q), _ptr(v))
    return v


def round_bf16(v):
    lib = _load()
    v = _c(np.asarray(v, np.float64).ravel(), np.float64)
    out = np.empty(v.shape, np.float64)
    lib.orc_round_bf16_array(v.size, _ptr(v), _ptr(out))
    return out


def e2m1_encode(v):
    lib = _load()
    v = _c(np.asarray(v, np.float32).ravel(), np.float32)
    q = np.empty(v.shape, np.uint8)
    lib.orc_e2m1_encode_array(v.size, _ptr(v), _ptr(q))
    return q


def e2m1_decode(q):
    lib = _load()
    q = _c(np.asarray(q, np.uint8).ravel(), np.uint8)
    v = np.empty(q.shape, np.float64)
    lib.orc_e2m1_decode_array(q.size, _ptr(q), _ptr(v))
    return v


def mx_exponent(amax, elem):
    return _load().orc_mx_exponent(float(amax), elem)


def mx_quant_rows(v, elem):
    """MX quantisation of an fp32 [rows x cols] matrix along its rows, blocks
    of 32.  Returns (codes uint8 [rows x cols], E8M0 scales uint8
    [rows x cols/32])."""
    lib = _load()
    v = _c(v, np.float32)
    rows, cols = v.shape
    if cols % 32:
        raise ValueError("MX rows need a multiple of 32 columns")
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 32), np.uint8)
    lib.orc_mx_quant_rows(rows, cols, elem, _ptr(v), _ptr(q), _ptr(s))
    return q, s
