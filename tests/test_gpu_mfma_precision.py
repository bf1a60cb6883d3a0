"""The accumulation rule of the FP8 MFMA that the hidden-row check's FP8 / MX
slack is derived from: of 1 + (K-1) products of 2^-j in one output element,
the small products that share a group of 8 consecutive k with the 1.0 are
dropped once j >= 14 (13 fractional bits after alignment) and all others
survive; the bf16 MFMA keeps every product down to fp32 resolution."""
import os
import subprocess

import pytest

from tests.hw import build as hw

pytestmark = pytest.mark.gpu


def _run():
    exe = hw.path("mfma_accumulation")
    if not os.path.exists(exe):
        pytest.fail("tests/hw/mfma_accumulation is not built (run the build entry point)")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    rows = {}
    for line in r.stdout.split("\n"):
        if line.strip():
            m, K, j, frac = line.split()
            rows[(m, int(j))] = (int(K), float(frac))
    return rows


def test_fp8_mfma_aligns_groups_of_eight_products_to_13_fractional_bits():
    rows = _run()
    print(rows, flush=True)
    for j in range(4, 19):
        K, frac = rows[("f8f6f4", j)]
        want = 1.0 if j <= 13 else (K - 1 - 7) / (K - 1)
        assert abs(frac - want) < 1e-6, (j, frac, want)
    for j in range(4, 24):
        K, frac = rows[("bf16", j)]
        assert abs(frac - 1.0) < 1e-6, (j, frac)
