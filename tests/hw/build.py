"""Build the hardware-characterisation programs of the test suite (hipcc,
gfx950).  Called by the build entry point; the GPU tests only run them."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROGRAMS = ["mfma_accumulation", "fp8_convert", "gemm_loop_bench", "mfma_rate", "stream_rate"]


def build() -> None:
    for name in PROGRAMS:
        src = os.path.join(HERE, name + ".hip")
        out = os.path.join(HERE, name)
        subprocess.run(["hipcc", "--offload-arch=gfx950", "-O2", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", src, "-o", out + ".tmp"], check=True)
        os.replace(out + ".tmp", out)


def path(name: str) -> str:
    return os.path.join(HERE, name)
