"""What bounds the grouped GEMM's bf16 main loop: the 256 x 256 block tile's
stage loop in isolation (tests/hw/gemm_loop_bench.hip), with its fragment
reads, its MFMAs and its stage DMA switched on one at a time.  The figures
are printed (run with -s to see them); the assertions only check that the
program ran and that the rates are in a plausible range, so that a broken
build of the probe is noticed."""
import re
import subprocess

import pytest

from tests.hw import build as hw

pytestmark = pytest.mark.gpu


def test_main_loop_microbenchmark_runs_and_reports():
    exe = hw.path("gemm_loop_bench")
    print("gemm loop microbenchmark", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    rows = {}
    for line in r.stdout.splitlines():
        m = re.match(r"mode (\d) (\S+)\s+clk_per_stage ([\d.]+) tflops (\d+) pct_of_peak ([\d.]+)",
                     line)
        if m:
            rows[m.group(2)] = (float(m.group(3)), float(m.group(5)))
    assert set(rows) == {"mfma_only", "reads_only", "reads_mfma", "reads_dma", "mfma_dma",
                         "reads_mfma_dma"}, rows
    # the MFMAs alone need 2048 clocks per stage (two waves per SIMD)
    assert 1900 < rows["mfma_only"][0] < 4000, rows
    assert rows["mfma_only"][1] > 60.0, rows
    # adding reads and DMA can only slow the loop down
    assert rows["reads_mfma_dma"][0] >= rows["mfma_only"][0] * 0.95, rows
