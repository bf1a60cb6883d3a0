"""Pins of the oracle's shared experts (every token, weight 1, after the
gate-weighted routed sum): dense brute force over every expert, a zero
routed down projection that leaves exactly the shared SwiGLU FFN (checked
against torch), and n_shared = 0 reproducing the routed-only layer."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ORC_BF16, ORC_F32, ORC_FP8
from test_oracle_forward import _dense_experts, _make


def _split(inp, E):
    """Treat experts E.. of a _make() set as shared ones: the gate keeps the
    first E columns."""
    out = dict(inp)
    out["gw"] = np.ascontiguousarray(inp["gw"][:, :E])
    out["gwv"] = np.ascontiguousarray(inp["gwv"][:, :E])
    return out


def _run(inp, k, act, wdt, n_shared):
    sc = inp["scales"]
    ne = inp["W1"].shape[0]
    return oracle.forward(inp["x"], inp["gw"], None, list(inp["W1"]), list(inp["W3"]),
                          list(inp["W2"]), k, act, wdt,
                          W1s=[sc["W1"][e] for e in range(ne)] if sc else None,
                          W3s=[sc["W3"][e] for e in range(ne)] if sc else None,
                          W2s=[sc["W2"][e] for e in range(ne)] if sc else None,
                          n_shared=n_shared)


@pytest.mark.parametrize("act,wdt,d,f", [(ORC_F32, ORC_F32, 32, 48),
                                         (ORC_BF16, ORC_BF16, 64, 64),
                                         (ORC_BF16, ORC_FP8, 256, 128)])
@pytest.mark.parametrize("n_shared", [1, 2])
def test_shared_experts_match_dense_brute_force(act, wdt, d, f, n_shared):
    T, E, k = 20, 6, 2
    inp = _split(_make(T, d, f, E + n_shared, k, act, wdt, seed=40 + act + wdt + n_shared), E)
    out, ids, w = _run(inp, k, act, wdt, n_shared)
    ys = _dense_experts(inp, act, wdt)  # every expert, routed and shared
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            assert ids[t, j] < E
            ref[t] += float(w[t, j]) * ys[ids[t, j], t]
        for s in range(n_shared):
            ref[t] += ys[E + s, t]
    rms = math.sqrt(float(np.mean(ref ** 2)))
    assert np.abs(out - ref).max() <= 1e-9 * rms


def test_zero_routed_down_projection_leaves_the_shared_ffn():
    T, d, f, E, k = 16, 32, 64, 4, 2
    inp = _split(_make(T, d, f, E + 1, k, ORC_F32, ORC_F32, seed=45), E)
    inp["W2"] = inp["W2"].copy()
    inp["W2"][:E] = 0
    out, _, _ = _run(inp, k, ORC_F32, ORC_F32, 1)
    x = torch.from_numpy(inp["xv"])
    W1, W3, W2 = (torch.from_numpy(inp[n + "v"][E]) for n in ("W1", "W3", "W2"))
    h = torch.nn.functional.silu(x @ W1) * (x @ W3)
    ref = (h.float().double() @ W2).numpy()
    assert np.abs(out - ref).max() <= 1e-12 * math.sqrt(float(np.mean(ref ** 2)))


def test_no_shared_expert_is_the_routed_layer():
    T, d, f, E, k = 12, 64, 64, 5, 2
    inp = _split(_make(T, d, f, E + 1, k, ORC_BF16, ORC_BF16, seed=46), E)
    with_list, ids_a, _ = _run(inp, k, ORC_BF16, ORC_BF16, 0)
    routed = dict(inp)
    for n in ("W1", "W3", "W2"):
        routed[n] = inp[n][:E]
    alone, ids_b, _ = _run(routed, k, ORC_BF16, ORC_BF16, 0)
    assert np.array_equal(with_list, alone) and np.array_equal(ids_a, ids_b)
