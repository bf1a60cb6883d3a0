"""Shared test utilities: tolerance checks and host-side views."""
from __future__ import annotations

import math

import numpy as np
import torch

# Output tolerance, relative to the RMS of the exact (unrounded) oracle output:
# bf16 layers 1e-2 (on the fp32-output run), FP8 and MXFP4 layers 5e-2, fp32
# layers 1e-4.
TOL = {0: 1e-4, 1: 1e-2, 2: 5e-2, 3: 5e-2}


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    rms = math.sqrt(float(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(out.astype(np.float64) - ref))) / rms


def check_output(out, ref: np.ndarray, bar: float, what: str = ""):
    """fp32 output: max|out-ref| <= bar*RMS.  bf16 output: every element within
    bar*RMS + half a bf16 ulp of the exact value (rounding a correct fp32
    result to bf16 alone costs up to half an ulp)."""
    if isinstance(out, torch.Tensor):
        is_bf16 = out.dtype == torch.bfloat16
        out = out.detach().float().cpu().numpy()
    else:
        is_bf16 = False
    out = out.astype(np.float64)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    diff = np.abs(out - ref)
    if is_bf16:
        lim = bar * rms + 0.5 * ulp_bf16(ref)
        bad = diff > lim
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond tolerance; "
                               f"worst excess {float((diff - lim).max()):.3e}, rms {rms:.3e}")
    else:
        err = float(diff.max()) / rms
        assert err <= bar, f"{what}: max err {err:.3e} x RMS > {bar}"
    return float(diff.max()) / rms


def f32_ulps(a: np.ndarray, b: np.ndarray) -> int:
    """Max distance in fp32 units-in-the-last-place between two fp32 arrays."""
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    return int(np.max(np.abs(ia - ib))) if ia.size else 0
