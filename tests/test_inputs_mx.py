"""The MXFP4 weight draw of the input module stores exactly the oracle's OCP
MX FP4 encoding of the same fp32 draws (packed K-major), so both sides of
every parity test read the same weights."""
import numpy as np
import torch

import oracle
from mixture_experts_layer_softmax_amd.configs import BF16, MXFP4, MoEConfig
from mixture_experts_layer_softmax_amd.inputs import make_inputs, mxfp4_quantize, unpack_mxfp4


def test_mxfp4_quantize_equals_oracle_encoding():
    g = torch.Generator().manual_seed(11)
    w = torch.randn((256, 96), generator=g) * 0.02
    w[32:64, 5] = 0.0                          # an all-zero block
    w[0:32, 7] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0] * 4)  # ties
    w[64:96, 9] = -w[64:96, 9]
    packed, scales = mxfp4_quantize(w)
    assert packed.shape == (96, 128) and scales.shape == (96, 8)
    codes = unpack_mxfp4(packed).numpy()
    q, s = oracle.mx_quant_rows(w.t().contiguous().numpy(), oracle.MX_E2M1)
    assert np.array_equal(codes, q) and np.array_equal(scales.numpy(), s)


def test_unpack_is_low_nibble_first():
    p = torch.tensor([[0x21, 0x43]], dtype=torch.uint8)
    assert unpack_mxfp4(p).tolist() == [[1, 2, 3, 4]]


def test_make_inputs_mxfp4_layout():
    cfg = MoEConfig("t", 8, 128, 256, 4, 2, BF16, MXFP4, BF16, n_shared=1)
    inp = make_inputs(cfg)
    assert inp["W1"].shape == (5, 256, 64) and inp["W1s"].shape == (5, 256, 4)
    assert inp["W2"].shape == (5, 128, 128) and inp["W2s"].shape == (5, 128, 8)
    assert inp["W1"].dtype == torch.uint8 and inp["W1s"].dtype == torch.uint8
