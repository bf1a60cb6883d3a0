"""Streaming rates of the chip's memory paths with nothing else running
(tests/hw/stream_rate.hip): HBM read through plain 16-byte vector loads and
through the direct-to-LDS buffer loads the GEMMs use, over 2 GiB (far
beyond L2 and the MALL), and the ds_read_b128 rate of one CU.  These are the
achievable rates the decode layers' HBM fractions are compared with.  The
figures are printed (run with -s to see them); the assertions only check
that the program ran and that the rates lie in a plausible range."""
import re
import subprocess

import pytest

from tests.hw import build as hw

pytestmark = pytest.mark.gpu


def test_memory_stream_rates():
    exe = hw.path("stream_rate")
    print("memory stream rates", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    tb = {m.group(1): float(m.group(2))
          for m in re.finditer(r"case (\S+)\s+bytes \d+ ms [\d.]+ tbps ([\d.]+)", r.stdout)}
    lds = re.search(r"case lds_read\s+bytes_per_clk_cu ([\d.]+)", r.stdout)
    assert "hbm_dma_lds" in tb and any(n.startswith("hbm_read_") for n in tb), r.stdout
    print("best plain-load read rate: %.3f TB/s" % max(v for n, v in tb.items()
                                                      if n.startswith("hbm_read_")), flush=True)
    assert lds is not None, r.stdout
    # HBM3E at 8 TB/s nominal: a stream reaches a good part of it and never
    # more; the LDS serves between 64 and 256 bytes per clock and CU
    for name, v in tb.items():
        assert 2.0 < v <= 8.0, (name, v)
    assert 64.0 <= float(lds.group(1)) <= 260.0, lds.group(0)
