"""Pins of the oracle's number formats against independent implementations:
torch's float8_e4m3fn and bfloat16 casts, and the format definitions."""
import numpy as np
import torch

import oracle


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


def test_e4m3_encode_matches_torch_on_every_bf16_value():
    # every finite bf16 value, clamped to the E4M3FN range (torch's cast is
    # round-to-nearest-even but not saturating, hence the clamp)
    v = _all_bf16_finite()
    ours = oracle.e4m3_encode(v)
    t = torch.from_numpy(v.copy()).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    ref = t.view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-3, 0.05, 1.0, 40.0, 300.0)])
    ours = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(ours, ref.numpy())


def test_e4m3_decode_and_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    nan = (codes & 0x7f) == 0x7f
    assert np.isnan(vals[nan]).all() and not np.isnan(vals[~nan]).any()
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(vals[~nan], ref[~nan])
    # definition: largest finite 448, smallest subnormal 2^-9, min normal 2^-6
    assert vals[0x7e] == 448.0 and vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    back = oracle.e4m3_encode(vals[~nan].astype(np.float32))
    assert np.array_equal(back, codes[~nan])


def test_e4m3_saturates_and_ties_to_even():
    v = np.array([448.0, 449.0, 500.0, 1e30, -1e30, 0.0, -0.0,
                  2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875], np.float32)
    q = oracle.e4m3_encode(v)
    assert list(q[:5]) == [0x7e, 0x7e, 0x7e, 0x7e, 0xfe]
    assert q[5] == 0x00 and q[6] == 0x80
    assert q[7] == 0x00  # 2^-10 is half the smallest subnormal: tie -> even (0)
    assert q[8] == 0x02  # 1.5 * 2^-9: tie between codes 1 and 2 -> 2
    assert q[9] == 0x38  # 1.0625 = 1 + 1/16 halfway 1 and 1.125 -> 1.0
    assert q[10] == 0x3a  # 1.1875 halfway 1.125 and 1.25 -> 1.25 (even mantissa)


def test_round_bf16_matches_torch_cast_of_fp32_values():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(300000) * s for s in (1e-30, 1e-3, 1.0, 1e20)])
    v32 = v.astype(np.float32)
    ours = oracle.round_bf16(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    # exact ties between two bf16 neighbours go to the even one
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7)])
    assert list(oracle.round_bf16(ties)) == [1.0, 1.0 + 2.0 ** -6, -2.0]


def test_round_bf16_of_fp64_is_single_rounding():
    # 1 + 2^-8 + 2^-40 is above the midpoint: a double rounding through fp32
    # would land on the tie and go down; one rounding goes up
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40])
    assert oracle.round_bf16(v)[0] == 1.0 + 2.0 ** -7


def test_fp8_group_quant_definition():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((5, 384)) * 3).astype(np.float32)
    v[1, 128:256] = 0.0  # an all-zero group takes scale 1
    v[2, :128] *= 1000.0
    q, s = oracle.fp8_quant_rows(v)
    assert q.shape == v.shape and s.shape == (5, 3)
    for r in range(5):
        for g in range(3):
            grp = v[r, g * 128:(g + 1) * 128]
            amax = np.float32(np.abs(grp).max())
            sc = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0))
            assert s[r, g] == sc
            ref = torch.from_numpy((grp / sc).astype(np.float32)).clamp(-448, 448)
            assert np.array_equal(q[r, g * 128:(g + 1) * 128],
                                  ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert s[1, 1] == 1.0 and not q[1, 128:256].any()
    # the group maximum maps to +-448 exactly
    i = np.argmax(np.abs(v[0, :128]))
    assert q[0, i] & 0x7f == 0x7e
