"""gfx950's packed FP8 conversion (v_cvt_pk_fp8_f32), applied after a clamp to
[-448, 448], against the oracle's OCP E4M3FN encoder (round to nearest even,
saturating at 448): the two must agree on every input the kernels convert,
so that the activation codes stay bit-exact when the kernels use the
instruction.  Inputs: every midpoint between adjacent E4M3 values and its
two fp32 neighbours, signed zeros, values beyond 448 and fp32 subnormals,
plus 2^22 seeded random bit patterns with magnitudes 2^-12 .. 2^10."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests.hw import build as hw

pytestmark = pytest.mark.gpu


def _inputs():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float64)
    pos = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    near = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)),
                           np.nextafter(m32, np.float32(0)), pos.astype(np.float32)])
    extra = np.array([0.0, 448.0, 448.5, 463.9, 464.0, 464.1, 480.0, 1e4, 3e38,
                      1e-40, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 2.0 ** -11], dtype=np.float32)
    rng = np.random.default_rng(7)
    e = rng.integers(127 - 12, 127 + 11, size=1 << 22).astype(np.uint32)
    m = rng.integers(0, 1 << 23, size=1 << 22).astype(np.uint32)
    rnd = ((e << 23) | m).view(np.float32)
    x = np.concatenate([near, extra, rnd])
    return np.concatenate([x, -x]).astype(np.float32)


def test_hardware_e4m3_conversion_equals_the_oracle_encoder():
    exe = hw.path("fp8_convert")
    if not os.path.exists(exe):
        pytest.fail("tests/hw/fp8_convert is not built (run the build entry point)")
    x = _inputs()
    with tempfile.TemporaryDirectory() as d:
        fin, fout = os.path.join(d, "in.f32"), os.path.join(d, "out.u8")
        x.tofile(fin)
        r = subprocess.run([exe, fin, fout], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        got = np.fromfile(fout, dtype=np.uint8)
    want = oracle.e4m3_encode(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]
