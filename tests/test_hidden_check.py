"""The hidden-row check of the GPU tests (tests/helpers.check_hidden_row)
accepts the oracle's own rounding of the exact SwiGLU output and rejects
planted mistakes: a code one step off away from a rounding boundary, a wrong
FP8 group scale or MX block exponent, a bf16 value one ulp off."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import check_hidden_row


def _exact(seed, f=512):
    rng = np.random.default_rng(seed)
    a, b = rng.standard_normal(f) * 1.7, rng.standard_normal(f) * 1.7
    return a / (1.0 + np.exp(-a)) * b


def _far_from_boundary(u, spacing):
    """Index of an element whose scaled value sits near a grid point."""
    frac = np.abs(u / spacing - np.round(u / spacing))
    return int(np.argmin(frac + (np.abs(u) < 1.0)))


def test_fp8_rows():
    h = _exact(1)
    q, s = oracle.fp8_quant_rows(h.astype(np.float32)[None, :])
    q, s = q[0], s[0]
    nf, ex = check_hidden_row(h, q, "fp8", s)
    assert nf == 0 and ex <= 1.0
    u = h / np.repeat(s.astype(np.float64), 128)
    i = _far_from_boundary(u, np.exp2(np.floor(np.log2(np.maximum(np.abs(u), 2 ** -6))) - 3))
    bad = q.copy()
    bad[i] = bad[i] + 1 if (bad[i] & 0x7F) < 0x7E else bad[i] - 1
    assert check_hidden_row(h, bad, "fp8", s)[1] > 1.0
    with pytest.raises(AssertionError):
        check_hidden_row(h, q, "fp8", s * np.float32(1.001))


def test_mx_rows():
    h = _exact(2, 256)
    q, x = oracle.mx_quant_rows(h.astype(np.float32)[None, :], oracle.MX_E4M3)
    q, x = q[0], x[0]
    nf, ex = check_hidden_row(h, q, "mx", x)
    assert nf == 0 and ex <= 1.0
    sc = np.exp2(np.repeat(x.astype(np.float64) - 127, 32))
    u = h / sc
    i = _far_from_boundary(u, np.exp2(np.floor(np.log2(np.maximum(np.abs(u), 2 ** -6))) - 3))
    bad = q.copy()
    bad[i] = bad[i] + 1 if (bad[i] & 0x7F) < 0x7E else bad[i] - 1
    assert check_hidden_row(h, bad, "mx", x)[1] > 1.0
    x2 = x.copy()
    x2[3] += 1
    with pytest.raises(AssertionError):
        check_hidden_row(h, q, "mx", x2)


def test_bf16_and_f32_rows():
    h = _exact(3)
    hb = torch.from_numpy(h).to(torch.bfloat16).double().numpy()
    nf, ex = check_hidden_row(h, hb, "bf16")
    assert nf == 0 and ex <= 1.0
    i = int(np.argmax(np.abs(h)))
    bad = hb.copy()
    bad[i] = hb[i] + 2.0 ** (np.floor(np.log2(abs(hb[i]))) - 7)  # one bf16 ulp
    assert check_hidden_row(h, bad, "bf16")[1] > 1.0
    h32 = h.astype(np.float32).astype(np.float64)
    assert check_hidden_row(h, h32, "f32")[1] <= 1.0
    off = h32.copy()
    off[i] *= 1.0 + 1e-4
    assert check_hidden_row(h, off, "f32")[1] > 1.0
