"""CPU oracle of the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports it and shares no code with it.
"""
from .oracle import (  # noqa: F401
    ORC_BF16,
    ORC_F32,
    ORC_FP8,
    ORC_MXFP4,
    MX_E2M1,
    MX_E4M3,
    build,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    expert_hidden,
    fp8_quant_rows,
    forward,
    mx_exponent,
    mx_quant_rows,
    permute,
    round_bf16,
    route,
)
