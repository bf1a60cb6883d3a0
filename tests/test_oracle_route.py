"""Pins of the oracle's gate: logits, top-k and renormalised softmax weights,
against independent definitions (exact rational arithmetic, brute force over
all k-subsets, closed forms)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import ORC_BF16, ORC_F32


def _bf16(a):
    """Round an fp32 array to bf16; return (uint16 bits, fp32 values)."""
    t = torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.float().numpy()


def _round_f32(fr: Fraction) -> float:
    """Exact round-to-nearest-even of a rational to fp32 (normal range)."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 23)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * q)


def _brute_topk(l, k):
    """The unique k-subset whose every member ranks before every non-member
    (larger logit, or equal logit and lower index), found by enumeration."""
    E = len(l)

    def before(a, b):
        return l[a] > l[b] or (l[a] == l[b] and a < b)

    found = [S for S in itertools.combinations(range(E), k)
             if all(before(a, b) for a in S for b in range(E) if b not in S)]
    assert len(found) == 1
    return sorted(found[0], key=lambda e: (-l[e], e))


def test_logits_fp32_exact_fma_chain():
    rng = np.random.default_rng(10)
    T, d, E = 3, 24, 5
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    logits, _, _ = oracle.route(x, w, bias, 2, ORC_F32)
    for t in range(T):
        for e in range(E):
            acc = 0.0
            for i in range(d):
                acc = _round_f32(Fraction(float(x[t, i])) * Fraction(float(w[i, e]))
                                 + Fraction(acc))
            acc = float(np.float32(np.float32(acc) + bias[e]))
            assert logits[t, e] == np.float32(acc), (t, e)


def test_logits_bf16_equal_sequential_fp32_sum():
    # bf16 x bf16 products are exact in fp32, so the fma chain equals a
    # sequential fp32 sum of exact products
    rng = np.random.default_rng(11)
    T, d, E = 40, 256, 16
    xb, xf = _bf16(rng.standard_normal((T, d)))
    wb, wf = _bf16(rng.standard_normal((d, E)) * 0.02)
    logits, _, _ = oracle.route(xb, wb, None, 4, ORC_BF16)
    acc = np.zeros((T, E), np.float32)
    for i in range(d):
        acc = (acc + xf[:, i:i + 1] * wf[i:i + 1, :]).astype(np.float32)
    assert np.array_equal(logits, acc)
    # a different order generally differs in the last bits: the order matters
    alt = (xf.astype(np.float32) @ wf.astype(np.float32)).astype(np.float32)
    assert np.abs(alt - acc).max() < 1e-4


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (10, 3)])
def test_topk_brute_force_random_and_ties(E, k):
    rng = np.random.default_rng(100 + E * 10 + k)
    T, d = 30, 16
    xb, _ = _bf16(rng.standard_normal((T, d)))
    wcols = rng.standard_normal((d, E)) * 0.02
    # exact ties: duplicate some gate columns (equal logits for every token)
    wcols[:, E - 1] = wcols[:, 0]
    if E > 3:
        wcols[:, 2] = wcols[:, 1]
    wb, _ = _bf16(wcols)
    logits, ids, w = oracle.route(xb, wb, None, k, ORC_BF16)
    for t in range(T):
        l = [float(v) for v in logits[t]]
        assert list(ids[t]) == _brute_topk(l, k)
        sel = np.array([l[e] for e in ids[t]], np.float64)
        u = np.exp(sel - sel.max())
        assert np.array_equal(w[t], (u / u.sum()).astype(np.float32))


def test_tie_lower_index_wins_and_zero_input():
    T, d, E, k = 4, 8, 6, 3
    xb, _ = _bf16(np.zeros((T, d)))
    wb, _ = _bf16(np.ones((d, E)))
    logits, ids, w = oracle.route(xb, wb, None, k, ORC_BF16)
    assert not logits.any()
    assert (ids == np.arange(k)).all()
    assert (w == np.float32(1.0 / k)).all()
    # all columns identical but non-zero: still indices 0..k-1 in order
    xb, _ = _bf16(np.ones((T, d)))
    _, ids, _ = oracle.route(xb, wb, None, k, ORC_BF16)
    assert (ids == np.arange(k)).all()


def test_bias_enters_selection_and_weights():
    T, d, E, k = 5, 8, 4, 2
    xb, _ = _bf16(np.zeros((T, d)))
    wb, _ = _bf16(np.zeros((d, E)))
    bias = np.array([0.0, 3.0, -1.0, 1.0], np.float32)
    logits, ids, w = oracle.route(xb, wb, bias, k, ORC_BF16)
    assert (logits == bias).all()
    assert (ids == [1, 3]).all()
    g0 = 1.0 / (1.0 + math.exp(-2.0))
    assert np.allclose(w[:, 0], g0, rtol=0, atol=1e-7) and np.allclose(w[:, 1], 1 - g0, atol=1e-7)


def test_weights_sum_to_one_and_k1():
    rng = np.random.default_rng(12)
    T, d, E = 200, 64, 32
    xb, _ = _bf16(rng.standard_normal((T, d)))
    wb, _ = _bf16(rng.standard_normal((d, E)) * 0.02)
    for k in (1, 2, 8, 32):
        _, ids, w = oracle.route(xb, wb, None, k, ORC_BF16)
        assert np.abs(w.astype(np.float64).sum(1) - 1.0).max() <= k * 2.0 ** -23
        assert (np.diff(w, axis=1) <= 0).all()  # descending logit -> descending weight
        assert all(len(set(r)) == k for r in ids)
        if k == 1:
            assert (w == 1.0).all()


def test_fp64_logits_agree_where_gap_exceeds_error_bound():
    # the selection must equal the exact-arithmetic selection wherever the
    # k-th/(k+1)-th gap exceeds the fp32 summation error bound
    rng = np.random.default_rng(13)
    T, d, E, k = 300, 512, 16, 2
    xb, xf = _bf16(rng.standard_normal((T, d)))
    wb, wf = _bf16(rng.standard_normal((d, E)) * 0.02)
    _, ids, _ = oracle.route(xb, wb, None, k, ORC_BF16)
    exact = xf.astype(np.float64) @ wf.astype(np.float64)
    bound = d * 2.0 ** -24 * (np.abs(xf).astype(np.float64) @ np.abs(wf).astype(np.float64))
    checked = 0
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-exact[t, e], e))
        gap = exact[t, order[k - 1]] - exact[t, order[k]]
        if gap > 2 * bound[t].max():
            assert set(ids[t]) == set(order[:k])
            checked += 1
    assert checked > T // 2
