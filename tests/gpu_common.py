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
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    B.moe_route(p, inp["x"], inp["gate_w"], inp.get("bias"), logits, ids, w)
    torch.cuda.synchronize()
    return logits, ids, w


def gpu_permute(cfg, ids, T=None, block_m=0):
    T = ids.shape[0] if T is None else T
    p = B.problem_of(cfg, T=T, block_m=block_m)
    dev = ids.device
    n = T * cfg.k
    out = {"counts": torch.empty(cfg.E, dtype=torch.int32, device=dev),
           "offsets": torch.empty(cfg.E + 1, dtype=torch.int32, device=dev),
           "slot_token": torch.empty(n, dtype=torch.int32, device=dev),
           "slot_k": torch.empty(n, dtype=torch.int32, device=dev),
           "token_slot": torch.empty(n, dtype=torch.int32, device=dev)}
    ws = B.alloc_workspace(p, dev)
    B.moe_permute(p, ids, out["counts"], out["offsets"], out["slot_token"], out["slot_k"],
                  out["token_slot"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
