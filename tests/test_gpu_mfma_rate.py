"""Register-only MFMA issue rates of the chip (tests/hw/mfma_rate.hip): the
matrix-core rate each MFMA form the library uses sustains with no memory
traffic, and the issue interval of a dependent chain (the bound of the gate's
sequential fp32 fma chain).  The figures are printed (run with -s to see
them); the assertions check that the program ran and that the rates lie in a
plausible range, so that a broken build of the probe is noticed."""
import re
import subprocess

import pytest

from tests.hw import build as hw

pytestmark = pytest.mark.gpu


def test_register_only_mfma_rates():
    exe = hw.path("mfma_rate")
    print("register-only MFMA rates", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    rows = {}
    for line in r.stdout.splitlines():
        m = re.match(r"case (\S+)\s+waves_per_simd (\d) chains (\d) clk_per_mfma ([\d.]+) "
                     r"flop_per_clk_cu (\d+)", line)
        if m:
            rows[m.group(1)] = (float(m.group(4)), float(m.group(5)))
    assert set(rows) == {"bf16_16x16x32", "fp8_16x16x128", "fp4xfp8_16x16x128",
                         "fp4xfp4_16x16x128", "f32_16x16x4", "bf16_chain", "f32_chain",
                         "f32_two_chains"}, rows
    # per-CU FLOP per clock against the nominal 4096 (bf16), 8192 (fp8 / fp4
    # forms) and 256 (fp32): independent chains reach most of it, and no form
    # exceeds twice its nominal rate
    for name, nominal in (("bf16_16x16x32", 4096), ("fp8_16x16x128", 8192),
                          ("fp4xfp8_16x16x128", 8192), ("f32_16x16x4", 256)):
        assert 0.5 * nominal < rows[name][1] <= 2.0 * nominal, (name, rows[name])
    # a dependent chain can only be slower than independent ones
    assert rows["f32_chain"][0] >= 0.95 * rows["f32_16x16x4"][0], rows
