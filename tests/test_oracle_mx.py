"""Pins of the oracle's OCP MX formats (E2M1 codes, E8M0 block exponents, MX
FP8/FP4 block quantisation) and of its MXFP4 layer forward.

The E2M1 value table is the FP4 element table of the OCP Microscaling
Formats (MX) v1.0 specification; the encoder is checked against
brute-force nearest-even search over that table, the E4M3 blocks against
torch's float8_e4m3fn cast, the block exponent against numpy's frexp, and the
layer against a dense fp64 evaluation that dequantises with independent numpy
code."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import MX_E2M1, MX_E4M3, ORC_BF16, ORC_MXFP4

# FP4 E2M1 magnitudes of codes 0..7 (OCP MX v1.0 FP4 element table)
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_brute(v):
    """Nearest E2M1 code by exhaustive search; ties to the even code; beyond
    6 saturates; the sign bit follows the sign of v (also for zero)."""
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.ravel()):
        a = min(abs(x), 6.0)
        d = np.abs(E2M1_TABLE - a)
        best = np.flatnonzero(d == d.min())
        code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
        out.ravel()[i] = code | (8 if math.copysign(1.0, x) < 0 else 0)
    return out


def _exp_np(amax, emax):
    """floor(log2(amax)) - emax via numpy frexp, clamped; 0 for zero."""
    m, e = np.frexp(np.asarray(amax, np.float64))
    x = np.clip(e.astype(np.int64) - 1 - emax, -127, 127)
    return np.where(np.asarray(amax) == 0, 0, x)


def test_e2m1_decode_is_the_spec_table():
    v = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(v[:8], E2M1_TABLE)
    assert np.array_equal(v[8:], -E2M1_TABLE)
    assert math.copysign(1.0, v[8]) < 0  # code 8 is -0


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(1)
    mids = (E2M1_TABLE[1:] + E2M1_TABLE[:-1]) / 2  # every tie point
    eps = np.float32(1e-6)
    v = np.concatenate([mids, mids + eps, mids - eps, E2M1_TABLE, [6.5, 7.0, 100.0, 1e30],
                        rng.uniform(0, 7, 4000), rng.standard_normal(2000) * 3]).astype(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.e2m1_encode(v), _e2m1_brute(v))


def test_e2m1_round_trip_of_every_code():
    v = oracle.e2m1_decode(np.arange(16)).astype(np.float32)
    assert np.array_equal(oracle.e2m1_encode(v), np.arange(16, dtype=np.uint8))


@pytest.mark.parametrize("elem,emax", [(MX_E2M1, 2), (MX_E4M3, 8)])
def test_block_exponent_rule(elem, emax):
    rng = np.random.default_rng(2)
    amax = np.concatenate([np.exp2(rng.uniform(-30, 30, 500)), np.exp2(np.arange(-20, 21)),
                           np.nextafter(np.exp2(np.arange(-20, 21)), 0), [0.0, 1e-40, 3e38]])
    amax = amax.astype(np.float32)
    got = np.array([oracle.mx_exponent(a, elem) for a in amax])
    assert np.array_equal(got, _exp_np(amax, emax))
    assert oracle.mx_exponent(4.0, MX_E2M1) == 0 and oracle.mx_exponent(3.99, MX_E2M1) == -1
    assert oracle.mx_exponent(256.0, MX_E4M3) == 0 and oracle.mx_exponent(255.9, MX_E4M3) == -1


def _blocks(seed, rows=24, cols=256):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-8, 8, (rows, 1)))).astype(np.float32)
    v[3, 32:64] = 0.0                     # an all-zero block
    v[5, 0:32] = 7.0                      # a constant block
    v[6, 64:96] = np.float32(2.0 ** -140)  # a subnormal block
    return v


def test_mx_fp8_blocks_match_torch_cast():
    v = _blocks(3)
    q, s = oracle.mx_quant_rows(v, MX_E4M3)
    blk = v.reshape(v.shape[0], -1, 32)
    x = _exp_np(np.abs(blk).max(axis=2), 8)
    assert np.array_equal(s.astype(np.int64), x + 127)
    scaled = torch.from_numpy(np.ldexp(blk.astype(np.float64), -x[:, :, None]).astype(np.float32))
    ref = scaled.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref.reshape(v.shape))


def test_mx_fp4_blocks_match_brute_force():
    v = _blocks(4, cols=128)
    q, s = oracle.mx_quant_rows(v, MX_E2M1)
    blk = v.reshape(v.shape[0], -1, 32)
    x = _exp_np(np.abs(blk).max(axis=2), 2)
    assert np.array_equal(s.astype(np.int64), x + 127)
    ref = _e2m1_brute(np.ldexp(blk.astype(np.float64), -x[:, :, None]))
    assert np.array_equal(q, ref.reshape(v.shape))


@pytest.mark.parametrize("elem,top", [(MX_E2M1, 4.0), (MX_E4M3, 256.0)])
def test_block_maximum_lands_in_the_top_binade(elem, top):
    # the scale puts each block's largest magnitude in [2^emax, 2^(emax+1)),
    # so its code is one of the format's largest values (saturation aside);
    # blocks whose exponent is clamped at -127 (tiny values) are exempt
    v = _blocks(5, cols=128)
    q, s = oracle.mx_quant_rows(v, elem)
    dec = oracle.e2m1_decode(q) if elem == MX_E2M1 else oracle.e4m3_decode(q)
    dec = np.abs(dec.reshape(v.shape[0], -1, 32)).max(axis=2)
    amax = np.abs(v.reshape(v.shape[0], -1, 32)).max(axis=2)
    clamped = s == 0
    assert clamped.sum() == 1 and amax[clamped][0] == np.float32(2.0 ** -140)
    assert ((dec >= top) | (amax == 0) | clamped).all()


def _mxfp4_weights(w):
    """[K x N] fp32 -> (codes [K x N], E8M0 [K/32 x N], values [K x N]) with
    blocks of 32 along K, by independent numpy code."""
    K, N = w.shape
    blk = w.reshape(K // 32, 32, N).astype(np.float64)
    x = _exp_np(np.abs(blk).max(axis=1).astype(np.float32), 2)  # [K/32 x N]
    codes = _e2m1_brute(np.ldexp(blk, -x[:, None, :])).reshape(K, N)
    mag = E2M1_TABLE[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    vals = np.ldexp(mag.reshape(K // 32, 32, N), x[:, None, :]).reshape(K, N)
    return codes, (x + 127).astype(np.uint8), vals


def _mx_fp8_dequant(v32):
    """Rows of fp32 -> MX FP8 (torch E4M3 cast, numpy exponent) -> fp64."""
    v = np.asarray(v32, np.float32)
    blk = v.reshape(v.shape[0], -1, 32)
    x = _exp_np(np.abs(blk).max(axis=2), 8)
    sc = torch.from_numpy(np.ldexp(blk.astype(np.float64), -x[:, :, None]).astype(np.float32))
    c = sc.clamp(-448, 448).to(torch.float8_e4m3fn).double().numpy()
    return np.ldexp(c, x[:, :, None]).reshape(v.shape)


def test_mxfp4_forward_matches_dense_brute_force():
    T, d, f, E, k = 20, 128, 96, 5, 2
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    gw = torch.from_numpy((rng.standard_normal((d, E)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    gwb = gw.view(torch.int16).numpy().view(np.uint16)
    W = {n: [_mxfp4_weights((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
             for _ in range(E)] for n, (K, N) in (("W1", (d, f)), ("W3", (d, f)), ("W2", (f, d)))}
    out, ids, w = oracle.forward(xb, gwb, None, [c for c, _, _ in W["W1"]],
                                 [c for c, _, _ in W["W3"]], [c for c, _, _ in W["W2"]], k,
                                 ORC_BF16, ORC_MXFP4, W1s=[s for _, s, _ in W["W1"]],
                                 W3s=[s for _, s, _ in W["W3"]], W2s=[s for _, s, _ in W["W2"]])
    xq = _mx_fp8_dequant(x.float().numpy())
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            a = xq[t] @ W["W1"][e][2]
            b = xq[t] @ W["W3"][e][2]
            h = a / (1.0 + np.exp(-a)) * b
            hq = _mx_fp8_dequant(h.astype(np.float32)[None, :])[0]
            ref[t] += float(w[t, j]) * (hq @ W["W2"][e][2])
    rms = math.sqrt(float(np.mean(ref ** 2)))
    assert np.abs(out - ref).max() <= 1e-9 * rms


def test_mxfp4_down_projection_block_sign_flip():
    # the output is linear in W2 for a fixed h: flipping the sign bit of the
    # first 32-row K block of W2 (one E8M0 scale row) changes the output by
    # exactly twice that block's contribution h[:, :32] @ W2[:32]
    T, d, f, E, k = 6, 64, 64, 1, 1
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    gwb = np.zeros((d, E), np.uint16)
    mk = lambda K, N: _mxfp4_weights((rng.standard_normal((K, N)) * 0.02).astype(np.float32))  # noqa: E731
    W1, W3, W2 = mk(d, f), mk(d, f), mk(f, d)
    args = dict(W1s=[W1[1]], W3s=[W3[1]], W2s=[W2[1]])
    out, _, _ = oracle.forward(xb, gwb, None, [W1[0]], [W3[0]], [W2[0]], k, ORC_BF16, ORC_MXFP4,
                               **args)
    neg = W2[0].copy()
    neg[:32] ^= 8  # flip the sign of the first K block of W2
    out2, _, _ = oracle.forward(xb, gwb, None, [W1[0]], [W3[0]], [neg], k, ORC_BF16, ORC_MXFP4,
                                **args)
    xq = _mx_fp8_dequant(x.float().numpy())
    h = (xq @ W1[2]) / (1.0 + np.exp(-(xq @ W1[2]))) * (xq @ W3[2])
    hq = _mx_fp8_dequant(h.astype(np.float32))
    part = hq[:, :32] @ W2[2][:32]
    assert np.abs(out - out2 - 2 * part).max() <= 1e-12 * np.abs(out).max()


def test_mxfp4_expert_hidden_is_dense_swiglu():
    # unrounded SwiGLU output of each token through one MXFP4 expert against
    # numpy matmuls on the MX FP8 activations and MX FP4 weights decoded by
    # independent code
    T, d, f = 10, 128, 64
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    W1 = _mxfp4_weights((rng.standard_normal((d, f)) * 0.02).astype(np.float32))
    W3 = _mxfp4_weights((rng.standard_normal((d, f)) * 0.02).astype(np.float32))
    xq = _mx_fp8_dequant(x.float().numpy())
    a, b = xq @ W1[2], xq @ W3[2]
    ref = a / (1.0 + np.exp(-a)) * b
    for t in range(T):
        h = oracle.expert_hidden(xb, t, W1[0], W3[0], ORC_BF16, ORC_MXFP4, W1s=W1[1], W3s=W3[1])
        assert np.abs(h - ref[t]).max() <= 1e-12 * np.abs(ref[t]).max()
