"""Helpers of the GPU parity tests: draw inputs on the GPU, hand the same
bits to the oracle, run the library through its C ABI."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from mixture_experts_layer_softmax_amd import binding as B
from mixture_experts_layer_softmax_amd.configs import BF16, F32, FP8, MXFP4
from mixture_experts_layer_softmax_amd.inputs import host_arrays, host_weight, make_inputs

ORC = {F32: oracle.ORC_F32, BF16: oracle.ORC_BF16, FP8: oracle.ORC_FP8, MXFP4: oracle.ORC_MXFP4}


def say(*a):
    print(*a, flush=True)


def poison_(t: torch.Tensor) -> torch.Tensor:
    """Fill every byte of t with 0xFF: NaN in fp32 and bf16, -1 in int32.  A
    kernel that skips an element it should write leaves NaN or -1 behind
    instead of a stale value from an earlier call in the same memory."""
    t.view(torch.uint8).fill_(0xFF)
    return t


def poisoned(shape, dtype, device="cuda") -> torch.Tensor:
    return poison_(torch.empty(shape, dtype=dtype, device=device))


def poisoned_workspace(p, device="cuda") -> torch.Tensor:
    return poison_(B.alloc_workspace(p, device))


def gpu_inputs(cfg, seed=None):
    inp = make_inputs(cfg, device="cuda", seed=seed)
    torch.cuda.synchronize()
    return inp


def oracle_route_rows(cfg, inp, rows):
    """Oracle gate for the listed token rows (numpy index array)."""
    x = host_arrays(inp["x"][torch.as_tensor(rows, device=inp["x"].device)])
    gw = host_arrays(inp["gate_w"])
    bias = None if inp.get("bias") is None else inp["bias"].cpu().numpy()
    return oracle.route(x, gw, bias, cfg.k, ORC[cfg.act_dtype])


def oracle_forward_rows(cfg, inp, rows):
    """Oracle forward of the listed token rows; copies only the experts those
    tokens route to (routing taken from the oracle's own gate) and the shared
    experts, which every token uses."""
    rows = np.asarray(rows, np.int64)
    _, ids, _ = oracle_route_rows(cfg, inp, rows)
    E = cfg.E
    need = sorted(set(int(e) for e in ids.reshape(-1))) + list(range(E, E + cfg.n_shared))
    W = {n: [None] * (E + cfg.n_shared) for n in ("W1", "W3", "W2", "W1s", "W3s", "W2s")}
    for e in need:
        for n in ("W1", "W3", "W2"):
            W[n][e], W[n + "s"][e] = host_weight(cfg, inp, n, e)
    x = host_arrays(inp["x"][torch.as_tensor(rows, device=inp["x"].device)])
    gw = host_arrays(inp["gate_w"])
    bias = None if inp.get("bias") is None else inp["bias"].cpu().numpy()
    sc = cfg.w_dtype in (FP8, MXFP4)
    out, ids, w = oracle.forward(x, gw, bias, W["W1"], W["W3"], W["W2"], cfg.k,
                                 ORC[cfg.act_dtype], ORC[cfg.w_dtype],
                                 W1s=W["W1s"] if sc else None, W3s=W["W3s"] if sc else None,
                                 W2s=W["W2s"] if sc else None, n_shared=cfg.n_shared)
    return out, ids, w


def gpu_route(cfg, inp, T=None):
    T = inp["x"].shape[0] if T is None else T
    p = B.problem_of(cfg, T=T)
    dev = inp["x"].device
    logits = poisoned((T, cfg.E), torch.float32, dev)
    ids = poisoned((T, cfg.k), torch.int32, dev)
    w = poisoned((T, cfg.k), torch.float32, dev)
    B.moe_route(p, inp["x"], inp["gate_w"], inp.get("bias"), logits, ids, w)
    torch.cuda.synchronize()
    return logits, ids, w


def gpu_permute(cfg, ids, T=None, block_m=0):
    T = ids.shape[0] if T is None else T
    p = B.problem_of(cfg, T=T, block_m=block_m)
    dev = ids.device
    n = T * cfg.k
    out = {"counts": poisoned(cfg.E, torch.int32, dev),
           "offsets": poisoned(cfg.E + 1, torch.int32, dev),
           "slot_token": poisoned(n, torch.int32, dev),
           "slot_k": poisoned(n, torch.int32, dev),
           "token_slot": poisoned(n, torch.int32, dev)}
    ws = poisoned_workspace(p, dev)
    B.moe_permute(p, ids, out["counts"], out["offsets"], out["slot_token"], out["slot_k"],
                  out["token_slot"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def forward(cfg, inp, packed, out_dtype=None, block_m=0, dbg=None, stream=None):
    """One moe_forward of cfg through the C ABI with a freshly allocated
    workspace and output whose every byte is 0xFF (NaN) beforehand.  packed
    None passes the weights in their stated layout (MOE_W_KN)."""
    T = inp["x"].shape[0]
    p = B.problem_of(cfg, T=T, block_m=block_m, out_dtype=out_dtype,
                     w_layout=B.MOE_W_KN if packed is None else B.MOE_W_NK)
    ws = poisoned_workspace(p, inp["x"].device)
    out = poison_(B.out_tensor(cfg, T=T, device=inp["x"].device, out_dtype=out_dtype))
    return B.forward(cfg, inp, packed, out=out, ws=ws, dbg=dbg, out_dtype=out_dtype,
                     block_m=block_m, stream=stream)


def forward_ring(cfg, inp, packed, ws=None, out=None, out_dtype=None, block_m=0, dbg=None,
                 stream=None):
    """moe_forward_ring through the C ABI; a workspace or output not passed in
    is allocated with every byte 0xFF (NaN) beforehand."""
    T = inp["x"].shape[0]
    p = B.problem_of(cfg, T=T, block_m=block_m, out_dtype=out_dtype)
    if ws is None:
        ws = poisoned(B.ring_workspace_size(p), torch.uint8, inp["x"].device)
    if out is None:
        out = poison_(B.out_tensor(cfg, T=T, device=inp["x"].device, out_dtype=out_dtype))
    return B.forward(cfg, inp, packed, out=out, ws=ws, dbg=dbg, out_dtype=out_dtype,
                     block_m=block_m, stream=stream, ring=True)


def debug_buffers(cfg, T=None, keys=None):
    """Poisoned device buffers for moe_debug's routing outputs."""
    T = cfg.T if T is None else T
    n = T * cfg.k
    sizes = {"topk_ids": n, "topk_w": n, "counts": cfg.E, "offsets": cfg.E + 1,
             "slot_token": n, "slot_k": n, "token_slot": n}
    keys = keys or list(sizes)
    return {k: poisoned(sizes[k], torch.float32 if k == "topk_w" else torch.int32)
            for k in keys}


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
