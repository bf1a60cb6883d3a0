"""MI355X-native MoE layer forward: softmax top-k gate, atomic-free expert
permutation, persistent grouped SwiGLU expert GEMMs on CDNA4 MFMA and a
deterministic gate-weighted combine, behind the C ABI of include/moe.h.

The compute lives in libmoe.so (HIP for gfx950); the Python side only
marshals arguments (binding.py) and draws seeded inputs (inputs.py).
"""
from .configs import CONFIGS, ORDER, MoEConfig  # noqa: F401
