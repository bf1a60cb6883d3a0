"""Build libmoe.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

Usage: python -m mixture_experts_layer_softmax_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.cpp", "route.hip", "permute.hip", "quant.hip", "gemm.hip", "combine.hip",
           "pack.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# per-source additions: the GEMM's work-queue atomic is issued by one lane
# and its result consumed a whole tile later, so the wave-aggregating atomic
# rewrite (which waits for the result at once) is switched off there
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *COMMON, *EXTRA.get(src, [])]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
