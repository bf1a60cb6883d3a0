"""The MoE-layer workloads this library is measured and checked on.

Each is a single-GPU layer forward.  Names say what the workload is; sizes are
tokens T, hidden d, expert intermediate f, experts E and top-k.
"""
from __future__ import annotations

from dataclasses import dataclass

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3  # same codes as moe_dtype in include/moe.h


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    act_dtype: int
    w_dtype: int
    out_dtype: int
    skew_bias: bool = False  # router bias_e = -1.2 ln(pi(e)+1)
    seed: int = 0
    n_shared: int = 0        # shared experts: every token, weight 1

    @property
    def slots(self) -> int:
        return self.T * self.k

    @property
    def expert_flops(self) -> float:
        """Algorithmic expert-GEMM FLOPs: 2 * T*(k + n_shared) * 3 * d * f."""
        return 2.0 * self.T * (self.k + self.n_shared) * 3 * self.d * self.f

    @property
    def router_flops(self) -> float:
        return 2.0 * self.T * self.d * self.E

    def replace(self, **kw) -> "MoEConfig":
        d = self.__dict__.copy()
        d.update(kw)
        return MoEConfig(**d)


CONFIGS = {
    # the five stated workloads
    "tiny_fp32": MoEConfig("tiny_fp32", 64, 128, 256, 8, 2, F32, F32, F32),
    "prefill_bf16": MoEConfig("prefill_bf16", 16384, 2048, 2048, 32, 2, BF16, BF16, BF16),
    "decode_bf16": MoEConfig("decode_bf16", 64, 7168, 2048, 256, 8, BF16, BF16, BF16),
    "skewed_bf16": MoEConfig("skewed_bf16", 8192, 4096, 1536, 64, 6, BF16, BF16, BF16,
                             skew_bias=True),
    "prefill_fp8": MoEConfig("prefill_fp8", 32768, 7168, 2048, 256, 8, BF16, FP8, BF16),
    # the prefill workload with one shared expert of the routed experts' shape
    # (the shared-expert phases of the MegaMoE-vs-MoE-systems page, section 2.7)
    "prefill_bf16_shared": MoEConfig("prefill_bf16_shared", 16384, 2048, 2048, 32, 2, BF16,
                                     BF16, BF16, n_shared=1),
    # the FP8 x FP4 expert variant (MX FP4 weights, MX FP8 activations) at
    # the FP8 prefill and the decode shapes
    "prefill_mxfp4": MoEConfig("prefill_mxfp4", 32768, 7168, 2048, 256, 8, BF16, MXFP4, BF16),
    "decode_mxfp4": MoEConfig("decode_mxfp4", 64, 7168, 2048, 256, 8, BF16, MXFP4, BF16),
}

ORDER = ["tiny_fp32", "prefill_bf16", "decode_bf16", "skewed_bf16", "prefill_fp8"]
