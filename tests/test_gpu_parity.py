"""GPU parity: libmoe.so (through its C ABI) against the CPU oracle.

Routing (logits, ids), histogram, offsets, permutation and FP8 activation
codes must be bit-exact; gate weights within 4 fp32 ulp; layer outputs
within the tolerance of the layer's precision (fp32 output: max error <=
bar x RMS; bf16 output: every element within bar x RMS + 1/2 bf16 ulp).
Every workspace, output and debug buffer is filled with 0xFF bytes (NaN,
or -1 for integers) before the call that writes it, so an element a kernel
fails to write cannot pass on a value left by an earlier call.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_softmax_amd import binding as B
from mixture_experts_layer_softmax_amd.configs import BF16, CONFIGS, F32, FP8, MXFP4, MoEConfig
from tests.gpu_common import (debug_buffers, forward, forward_ring, free, gpu_inputs, gpu_permute, gpu_route,
                              oracle_forward_rows, oracle_route_rows, poison_, poisoned,
                              poisoned_workspace, say)
from tests.helpers import TOL, check_hidden_row, check_output, f32_ulps

pytestmark = pytest.mark.gpu

# Reduced shapes of the five workloads: the oracle checks every output, the
# expert tiles are several per expert and the last one is ragged.
REDUCED = {
    "tiny_fp32": CONFIGS["tiny_fp32"],
    "prefill_bf16_r": MoEConfig("prefill_bf16_r", 1000, 512, 512, 32, 2, BF16, BF16, BF16),
    "decode_bf16_r": MoEConfig("decode_bf16_r", 16, 1024, 512, 64, 8, BF16, BF16, BF16),
    "skewed_bf16_r": MoEConfig("skewed_bf16_r", 600, 512, 384, 64, 6, BF16, BF16, BF16,
                               skew_bias=True),
    "prefill_fp8_r": MoEConfig("prefill_fp8_r", 300, 512, 256, 16, 8, BF16, FP8, BF16),
    "prefill_mxfp4_r": MoEConfig("prefill_mxfp4_r", 300, 512, 256, 16, 8, BF16, MXFP4, BF16),
    "decode_mxfp4_r": MoEConfig("decode_mxfp4_r", 16, 1024, 512, 64, 8, BF16, MXFP4, BF16),
}


def _forward(cfg, inp, out_dtype=None, block_m=0, dbg=None, packed=None):
    packed = B.pack_weights(inp) if packed is None else packed
    out = forward(cfg, inp, packed, out_dtype=out_dtype, block_m=block_m, dbg=dbg)
    torch.cuda.synchronize()
    return out


def _outputs_ok(cfg, out, ref, tag):
    bar = TOL[cfg.w_dtype]
    return check_output(out, ref, bar, f"{cfg.name} {tag}")


@pytest.mark.parametrize("name", list(REDUCED))
def test_route_bit_exact(name):
    cfg = REDUCED[name]
    say("route", name)
    inp = gpu_inputs(cfg)
    logits, ids, w = gpu_route(cfg, inp)
    ref_l, ref_ids, ref_w = oracle_route_rows(cfg, inp, np.arange(cfg.T))
    assert np.array_equal(logits.cpu().numpy(), ref_l)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert f32_ulps(w.cpu().numpy(), ref_w) <= 4


@pytest.mark.parametrize("E,k,act,d", [(20, 1, BF16, 128), (32, 2, BF16, 128), (40, 3, F32, 128),
                                       (256, 8, BF16, 128), (200, 5, BF16, 128),
                                       (256, 9, BF16, 128), (32, 2, BF16, 160), (256, 8, BF16, 96)])
def test_route_large_T_bit_exact(E, k, act, d):
    # T >= 16384: the gate runs the top-k inside the logits workgroup when
    # E <= 256 and k <= 8 (and a separate top-k kernel otherwise); duplicated
    # gate columns make exact logit ties, which must go to the lower index;
    # d = 160 and 96 end on a partial hidden chunk
    cfg = MoEConfig("route_T", 16400, d, 128, E, k, act, act, act)
    say("route large T", E, k, act, d)
    inp = gpu_inputs(cfg)
    inp["gate_w"][:, 7] = inp["gate_w"][:, 3]
    inp["gate_w"][:, E - 1] = inp["gate_w"][:, 0]
    logits, ids, w = gpu_route(cfg, inp)
    ref_l, ref_ids, ref_w = oracle_route_rows(cfg, inp, np.arange(cfg.T))
    assert np.array_equal(logits.cpu().numpy(), ref_l)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert f32_ulps(w.cpu().numpy(), ref_w) <= 4
    assert (ref_ids == 3).any() and not ((ref_ids == 7) & ~(ref_ids == 3).any(1)[:, None]).any()


@pytest.mark.parametrize("E,k,act", [(40, 3, BF16), (64, 6, BF16), (64, 8, BF16), (48, 2, F32)])
def test_route_mid_T_bit_exact(E, k, act):
    # 8192 <= T < 16384 with 33..64 experts (the skewed workload's regime):
    # experts split over two workgroups, then the top-k kernel; exact ties as
    # above
    cfg = MoEConfig("route_mid", 9000, 128, 128, E, k, act, act, act)
    say("route mid T", E, k, act)
    inp = gpu_inputs(cfg)
    inp["gate_w"][:, 7] = inp["gate_w"][:, 3]
    inp["gate_w"][:, E - 1] = inp["gate_w"][:, 0]
    logits, ids, w = gpu_route(cfg, inp)
    ref_l, ref_ids, ref_w = oracle_route_rows(cfg, inp, np.arange(cfg.T))
    assert np.array_equal(logits.cpu().numpy(), ref_l)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert f32_ulps(w.cpu().numpy(), ref_w) <= 4


@pytest.mark.parametrize("E,k", [(300, 8), (512, 33), (1000, 64), (1024, 70)])
def test_route_wide_E_bit_exact(E, k):
    # E above 256: the separate top-k kernel with 8 or 16 logits per lane,
    # k above one wave's 64 selections included; exact ties as above
    cfg = MoEConfig("route_E", 70, 128, 128, E, k, BF16, BF16, BF16)
    say("route wide E", E, k)
    inp = gpu_inputs(cfg)
    inp["gate_w"][:, 7] = inp["gate_w"][:, 3]
    inp["gate_w"][:, E - 1] = inp["gate_w"][:, 0]
    logits, ids, w = gpu_route(cfg, inp)
    ref_l, ref_ids, ref_w = oracle_route_rows(cfg, inp, np.arange(cfg.T))
    assert np.array_equal(logits.cpu().numpy(), ref_l)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert f32_ulps(w.cpu().numpy(), ref_w) <= 4


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("block_m", [0, 16, 128])
def test_permute_bit_exact(name, block_m):
    cfg = REDUCED[name]
    say("permute", name, block_m)
    inp = gpu_inputs(cfg)
    _, ids, _ = gpu_route(cfg, inp)
    got = gpu_permute(cfg, ids, block_m=block_m)
    ref = oracle.permute(ids.cpu().numpy(), cfg.E)
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("name", list(REDUCED))
def test_forward_parity_reduced(name):
    cfg = REDUCED[name]
    say("forward", name)
    inp = gpu_inputs(cfg)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    if cfg.w_dtype == BF16:
        out32 = _forward(cfg, inp, out_dtype=F32)
        _outputs_ok(cfg, out32, ref, "fp32 out")
    out = _forward(cfg, inp)
    _outputs_ok(cfg, out, ref, "native out")


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_bf16_r", "prefill_fp8_r",
                                  "prefill_mxfp4_r"])
def test_forward_every_tile_height(name, block_m):
    cfg = REDUCED[name]
    say("forward bm", name, block_m)
    inp = gpu_inputs(cfg)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    out = _forward(cfg, inp, out_dtype=F32, block_m=block_m)
    _outputs_ok(cfg, out, ref, f"bm={block_m}")


@pytest.mark.parametrize("log2_scale", [12, -12])
@pytest.mark.parametrize("name", ["prefill_bf16_r", "prefill_fp8_r"])
def test_expert_outputs_far_outside_fp16_range(name, log2_scale):
    # x times 2^s (exact in bf16) scales h and the expert outputs Y by about
    # 2^2s: near 2^24 their magnitudes lie far above fp16's largest finite
    # value, near 2^-24 far below its smallest normal one.  Y is stored as
    # fp16 codes under a power-of-two scale per 32 columns, which must keep
    # both within the layer's bar (relative to the output RMS).
    cfg = REDUCED[name]
    say("fp16 Y range", name, log2_scale)
    inp = gpu_inputs(cfg)
    inp["x"] = inp["x"] * (2.0 ** log2_scale)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    amax = float(np.abs(ref).max())
    assert (amax > 2.0 ** 20) if log2_scale > 0 else (amax < 2.0 ** -14), amax  # the premise
    out32 = _forward(cfg, inp, out_dtype=F32)
    _outputs_ok(cfg, out32, ref, f"x * 2^{log2_scale}, fp32 out")


@pytest.mark.parametrize("E,K,N,dt", [(3, 130, 70, torch.uint8), (2, 64, 4100, torch.int16),
                                      (1, 1000, 33, torch.int32), (5, 1, 1, torch.int16),
                                      (4, 7168, 256, torch.int16)])
def test_pack_weight_is_the_transpose(E, K, N, dt):
    # moe_pack_weight is pure data movement: [E][K][N] -> [E][N][K], bit for
    # bit, for 1-, 2- and 4-byte elements and ragged 64 x 64 tiles
    say("pack", E, K, N, dt)
    g = torch.Generator(device="cuda")
    g.manual_seed(K * 31 + N)
    info = torch.iinfo(dt)
    src = torch.randint(info.min, info.max, (E, K, N), generator=g, device="cuda", dtype=torch.int64
                        ).to(dt)
    dst = torch.full((E, N, K), -1, dtype=dt, device="cuda")
    B.moe_pack_weight(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src.cpu().transpose(1, 2).contiguous())


def test_route_logits_in_the_workspace():
    # moe_route with logits == NULL keeps them in the workspace: the same ids
    # and weights, bit for bit, as with a caller's logits buffer
    cfg = REDUCED["skewed_bf16_r"]
    say("route ws", cfg.name)
    inp = gpu_inputs(cfg)
    _, ids, w = gpu_route(cfg, inp)
    p = B.problem_of(cfg)
    ids2 = torch.full_like(ids, -1)
    w2 = torch.full_like(w, -1.0)
    ws = poisoned_workspace(p)
    B.moe_route(p, inp["x"], inp["gate_w"], inp.get("bias"), None, ids2, w2, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids) and torch.equal(w2, w)
    with pytest.raises(B.MoEError, match="WORKSPACE_TOO_SMALL"):
        B.moe_route(p, inp["x"], inp["gate_w"], inp.get("bias"), None, ids2, w2, ws=ws[:16])


def test_quantize_fp8_bit_exact():
    say("quant fp8")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = (torch.randn((333, 1024), generator=g, device="cuda") *
         torch.logspace(-3, 3, 1024, device="cuda")).to(torch.bfloat16)
    x[7, 128:256] = 0  # an all-zero group
    q = poisoned(x.shape, torch.uint8)
    s = poisoned((333, 8), torch.float32)
    B.moe_quantize_fp8(x, q, s)
    torch.cuda.synchronize()
    rq, rs = oracle.fp8_quant_rows(x.float().cpu().numpy())
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("name", ["prefill_fp8_r", "prefill_mxfp4_r", "fp8_small", "mx_small",
                                  "wide_fp8", "prefill_fp8", "prefill_mxfp4"])
def test_forward_activation_codes_bit_exact(name):
    # the gate quantises x for the FP8 / MXFP4 expert GEMMs in its own pass
    # over x: the codes and scales the fused call used equal the oracle's
    # quantisation of x, bit for bit, on every token
    cfg = REDUCED.get(name) or EDGE.get(name) or CONFIGS[name]
    say("fused x quantisation", name)
    inp = gpu_inputs(cfg)
    mx = cfg.w_dtype == MXFP4
    dbg = {"x_codes": poisoned((cfg.T, cfg.d), torch.uint8),
           "x_scales": poisoned((cfg.T, cfg.d // 32), torch.uint8) if mx
           else poisoned((cfg.T, cfg.d // 128), torch.float32)}
    _forward(cfg, inp, dbg=dbg)
    xf = inp["x"].float().cpu().numpy()
    if mx:
        rq, rs = oracle.mx_quant_rows(xf, oracle.MX_E4M3)
    else:
        rq, rs = oracle.fp8_quant_rows(xf)
    assert np.array_equal(dbg["x_codes"].cpu().numpy(), rq)
    assert np.array_equal(dbg["x_scales"].cpu().numpy(), rs)
    del inp, dbg
    free()


def test_quantize_mx_bit_exact():
    say("quant mx")
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    x = (torch.randn((333, 1024), generator=g, device="cuda") *
         torch.logspace(-3, 3, 1024, device="cuda")).to(torch.bfloat16)
    x[7, 128:160] = 0  # an all-zero block
    x[9, 0:32] = 3.0   # a constant block
    q = poisoned(x.shape, torch.uint8)
    s = poisoned((333, 32), torch.uint8)
    B.moe_quantize_mx(x, q, s)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quant_rows(x.float().cpu().numpy(), oracle.MX_E4M3)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy(), rs)


EDGE = {
    "T1": MoEConfig("T1", 1, 256, 128, 8, 2, BF16, BF16, BF16),
    "ragged": MoEConfig("ragged", 37, 128, 192, 4, 3, BF16, BF16, BF16),
    "many_empty": MoEConfig("many_empty", 3, 256, 128, 256, 2, BF16, BF16, BF16),
    "k1": MoEConfig("k1", 130, 128, 128, 8, 1, BF16, BF16, BF16),
    "k_eq_E": MoEConfig("k_eq_E", 40, 128, 128, 8, 8, BF16, BF16, BF16),
    "fp32_small": MoEConfig("fp32_small", 50, 32, 64, 3, 2, F32, F32, F32),
    "fp8_small": MoEConfig("fp8_small", 20, 128, 128, 4, 2, BF16, FP8, BF16),
    "mx_small": MoEConfig("mx_small", 20, 128, 128, 4, 2, BF16, MXFP4, BF16),
    "mx_T1": MoEConfig("mx_T1", 1, 256, 384, 8, 2, BF16, MXFP4, BF16),
    # hidden sizes above 8192: the combine takes a second pass over the row
    # (1024 lanes of 8 columns) and the gate a partial last chunk
    "wide_d": MoEConfig("wide_d", 9, 8256, 64, 4, 2, BF16, BF16, BF16),
    "wide_fp8": MoEConfig("wide_fp8", 7, 8320, 128, 4, 2, BF16, FP8, BF16),
    # the most experts a problem may have (1024), and a top-k of 64 (eight
    # groups of slot loads per combine lane)
    "E_max": MoEConfig("E_max", 300, 128, 128, 1024, 8, BF16, BF16, BF16),
    "k64": MoEConfig("k64", 50, 128, 64, 128, 64, BF16, BF16, BF16),
}


# the largest operands the 32-bit byte offsets of the GEMM loads allow: h
# (T*k rows of f bf16) and x (T rows of d bf16) each one row short of 2^31
# bytes (one more token is MOE_ERR_UNSUPPORTED, checked in test_abi)
MAX_OFFSET = {
    "max_h": MoEConfig("max_h", 65535, 256, 16384, 8, 1, BF16, BF16, BF16),
    "max_x": MoEConfig("max_x", 131071, 8192, 64, 4, 1, BF16, BF16, BF16),
}


@pytest.mark.parametrize("name", list(MAX_OFFSET))
def test_largest_supported_operands(name):
    cfg = MAX_OFFSET[name]
    say("max offsets", name)
    assert max(cfg.T * cfg.k * cfg.f, cfg.T * cfg.d) * 2 >= (1 << 31) - 2 * max(cfg.f, cfg.d)
    inp = gpu_inputs(cfg)
    dbg = debug_buffers(cfg, keys=["topk_ids"])
    out = _forward(cfg, inp, dbg=dbg)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(cfg.T, size=12, replace=False))
    rows[0], rows[-1] = 0, cfg.T - 1  # the last token's rows sit at the top of x and h
    ref, ref_ids, _ = oracle_forward_rows(cfg, inp, rows)
    assert np.array_equal(dbg["topk_ids"].view(cfg.T, cfg.k).cpu().numpy()[rows], ref_ids)
    _outputs_ok(cfg, out[torch.as_tensor(rows, device="cuda")], ref, "sampled")
    del inp, out
    free()


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_shapes(name):
    cfg = EDGE[name]
    say("edge", name)
    inp = gpu_inputs(cfg)
    _, ids, _ = gpu_route(cfg, inp)
    _, ref_ids, _ = oracle_route_rows(cfg, inp, np.arange(cfg.T))
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    _outputs_ok(cfg, _forward(cfg, inp, out_dtype=F32), ref, "fp32 out")
    _outputs_ok(cfg, _forward(cfg, inp), ref, "native out")


def test_all_tokens_to_one_expert():
    cfg = MoEConfig("hot", 300, 256, 128, 16, 1, BF16, BF16, BF16)
    say("hot expert")
    inp = gpu_inputs(cfg)
    inp["bias"] = torch.full((cfg.E,), -50.0, device="cuda")
    inp["bias"][5] = 50.0
    ref, ref_ids, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    assert (ref_ids == 5).all()
    _outputs_ok(cfg, _forward(cfg, inp, out_dtype=F32), ref, "fp32 out")


def test_forward_routing_equals_route_and_permute():
    # scheduling never changes routing: the fused call's routing is the
    # separate route + permute calls' routing, bit for bit
    cfg = REDUCED["skewed_bf16_r"]
    say("routing consistency")
    inp = gpu_inputs(cfg)
    dbg = debug_buffers(cfg)
    _forward(cfg, inp, dbg=dbg)
    _, ids, w = gpu_route(cfg, inp)
    assert torch.equal(dbg["topk_ids"].view(cfg.T, cfg.k), ids)
    assert torch.equal(dbg["topk_w"].view(cfg.T, cfg.k), w)
    perm = gpu_permute(cfg, ids)
    for key, v in perm.items():
        assert np.array_equal(dbg[key].cpu().numpy(), v), key


def test_forward_is_deterministic():
    cfg = REDUCED["skewed_bf16_r"]
    say("determinism")
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    outs = [forward(cfg, inp, packed, out_dtype=F32) for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_concurrent_calls_on_two_streams():
    # the library keeps no per-call state outside the workspace: two layers
    # (different shapes, dtypes and workspaces) enqueued alternately on two
    # streams give the same bits as when run one after the other
    cfgs = [REDUCED["skewed_bf16_r"], REDUCED["prefill_mxfp4_r"]]
    say("two streams", [c.name for c in cfgs])
    inps = [gpu_inputs(c) for c in cfgs]
    packs = [B.pack_weights(i) for i in inps]
    ref = [forward(c, i, p, out_dtype=F32) for c, i, p in zip(cfgs, inps, packs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for rep in range(3):
        for j in (0, 1):
            with torch.cuda.stream(streams[j]):
                outs[j].append(forward(cfgs[j], inps[j], packs[j], out_dtype=F32,
                                       stream=streams[j]))
    torch.cuda.synchronize()
    for j in (0, 1):
        for o in outs[j]:
            assert torch.equal(o, ref[j]), (cfgs[j].name)


def test_gemm_clock_record():
    """moe_debug.gemm_clock receives, per GEMM launch, the shader-clock and
    100 MHz reference ticks of the first workgroup; the implied clock lies in
    the chip's range, and recording it leaves the output unchanged."""
    cfg = REDUCED["prefill_bf16_r"]
    say("gemm clock")
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    ref = forward(cfg, inp, packed, out_dtype=F32)
    clock = torch.zeros(4, dtype=torch.int64, device="cuda")
    got = forward(cfg, inp, packed, out_dtype=F32, dbg={"gemm_clock": clock})
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    c = clock.cpu().tolist()
    for i in range(2):
        assert c[2 * i] > 0 and c[2 * i + 1] > 0, c
        mhz = 100.0 * c[2 * i] / c[2 * i + 1]
        assert 200.0 < mhz < 3000.0, (i, mhz, c)


# ---------------------------------------------------------------------------
# shared experts: every token, weight 1, after the routed sum
# ---------------------------------------------------------------------------

SHARED = {
    "sh_fp32": CONFIGS["tiny_fp32"].replace(name="sh_fp32", n_shared=1),
    "sh_bf16": REDUCED["prefill_bf16_r"].replace(name="sh_bf16", n_shared=2),
    "sh_decode": REDUCED["decode_bf16_r"].replace(name="sh_decode", n_shared=1),
    "sh_fp8": REDUCED["prefill_fp8_r"].replace(name="sh_fp8", n_shared=1),
    "sh_T1": EDGE["T1"].replace(name="sh_T1", n_shared=3),
    "sh_ragged": EDGE["ragged"].replace(name="sh_ragged", n_shared=1),
    "sh_mx": REDUCED["prefill_mxfp4_r"].replace(name="sh_mx", n_shared=1),
}


@pytest.mark.parametrize("name", list(SHARED))
def test_shared_expert_parity(name):
    cfg = SHARED[name]
    say("shared", name)
    inp = gpu_inputs(cfg)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    if cfg.w_dtype == BF16:
        _outputs_ok(cfg, _forward(cfg, inp, out_dtype=F32), ref, "fp32 out")
    _outputs_ok(cfg, _forward(cfg, inp), ref, "native out")


@pytest.mark.parametrize("block_m", [16, 64, 256])
def test_shared_expert_tile_heights(block_m):
    cfg = SHARED["sh_bf16"]
    say("shared bm", block_m)
    inp = gpu_inputs(cfg)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    _outputs_ok(cfg, _forward(cfg, inp, out_dtype=F32, block_m=block_m), ref, f"bm={block_m}")


def test_shared_expert_leaves_routing_alone():
    # the shared experts change neither the routing nor its permutation, and
    # the routed part of the output is the n_shared = 0 layer's
    cfg = SHARED["sh_bf16"]
    plain = cfg.replace(n_shared=0)
    say("shared routing")
    inp = gpu_inputs(cfg)
    keys = ("topk_ids", "counts", "offsets", "slot_token", "slot_k", "token_slot")
    dbgs = []
    for c in (cfg, plain):
        dbg = debug_buffers(c, keys=keys)
        _forward(c, inp, dbg=dbg)
        dbgs.append(dbg)
    for key in keys:
        assert torch.equal(dbgs[0][key], dbgs[1][key]), key


# ---------------------------------------------------------------------------
# full-size workloads in the launch configuration the benchmark times:
# routing (logits, ids, weights) of every token through moe_route, the fused
# call's routing and permutation of every token, and the outputs of a token
# sample the oracle computes one by one -- both with the fp32 output (the
# primary bar) and with the workload's own output type
# ---------------------------------------------------------------------------

FULL_SAMPLE = {"prefill_bf16": 256, "decode_bf16": 64, "skewed_bf16": 256, "prefill_fp8": 64,
               "prefill_bf16_shared": 256, "prefill_mxfp4": 64, "decode_mxfp4": 64}


HIDDEN = {n: REDUCED[n] for n in ("tiny_fp32", "prefill_bf16_r", "decode_bf16_r",
                                    "prefill_fp8_r", "prefill_mxfp4_r", "decode_mxfp4_r")}
HIDDEN.update({n: SHARED[n] for n in ("sh_fp32", "sh_bf16", "sh_fp8", "sh_mx")})


@pytest.mark.parametrize("name", list(HIDDEN) + ["prefill_bf16", "prefill_fp8", "prefill_mxfp4"])
def test_hidden_rows_match_oracle(name):
    """The W2 GEMM's input rows (SwiGLU output as stored: bf16 / fp32 values,
    or E4M3 codes with their FP8 group scales / MX block exponents) against
    the oracle's exact SwiGLU output of the same (token, expert): each element
    a correct rounding of a value within a small slack of the exact one.
    Reduced shapes: every slot; full sizes: sampled slots."""
    full = name not in HIDDEN
    cfg = CONFIGS[name] if full else HIDDEN[name]
    say("hidden", name)
    T, E, k, f = cfg.T, cfg.E, cfg.k, cfg.f
    rows, n = T * (k + cfg.n_shared), T * k
    q8 = cfg.w_dtype in (FP8, MXFP4)
    hdt = torch.uint8 if q8 else (torch.float32 if cfg.act_dtype == F32 else torch.bfloat16)
    dbg = debug_buffers(cfg, keys=["topk_ids", "slot_token", "slot_k"])
    dbg["h"] = poisoned((rows, f), hdt)
    if q8:
        dbg["h_scales"] = poisoned((rows, f // 128), torch.float32) if cfg.w_dtype == FP8 else \
            poisoned((rows, f // 32), torch.uint8)
    inp = gpu_inputs(cfg)
    _forward(cfg, inp, dbg=dbg)
    ids = dbg["topk_ids"].cpu().numpy()
    st, sk = dbg["slot_token"].cpu().numpy(), dbg["slot_k"].cpu().numpy()
    rng = np.random.default_rng(5)
    slots = np.sort(rng.choice(n, size=24, replace=False)) if full else np.arange(n)
    shared = [n + j * T + t for j in range(cfg.n_shared)
              for t in (rng.choice(T, size=4, replace=False) if full else range(T))]
    slots = np.concatenate([slots, np.asarray(shared, np.int64)]).astype(np.int64)
    pairs = []
    for s_ in slots:
        if s_ < n:
            t = int(st[s_])
            pairs.append((t, int(ids[t * k + int(sk[s_])])))
        else:
            pairs.append((int((s_ - n) % T), E + int((s_ - n) // T)))
    toks = sorted(set(t for t, _ in pairs))
    xi = {t: i for i, t in enumerate(toks)}
    from mixture_experts_layer_softmax_amd.inputs import host_arrays, host_weight
    xh = host_arrays(inp["x"][torch.as_tensor(toks, device="cuda")])
    sel = torch.as_tensor(slots, device="cuda")
    h = dbg["h"][sel]
    h = (h.float() if not q8 else h).cpu().numpy()
    hs = dbg["h_scales"][sel].cpu().numpy() if q8 else None
    fmt = {FP8: "fp8", MXFP4: "mx"}.get(cfg.w_dtype, "f32" if cfg.act_dtype == F32 else "bf16")
    orc = {F32: oracle.ORC_F32, BF16: oracle.ORC_BF16, FP8: oracle.ORC_FP8,
           MXFP4: oracle.ORC_MXFP4}
    wcache, flips, worst = {}, 0, 0.0
    for i, (t, e) in enumerate(pairs):
        if e not in wcache:
            wcache = {e: (host_weight(cfg, inp, "W1", e), host_weight(cfg, inp, "W3", e))}
        (w1, s1), (w3, s3) = wcache[e]
        exact = oracle.expert_hidden(xh, xi[t], w1, w3, orc[cfg.act_dtype], orc[cfg.w_dtype],
                                     W1s=s1, W3s=s3)
        nf, ex = check_hidden_row(exact, h[i], fmt, None if hs is None else hs[i])
        flips += nf
        worst = max(worst, ex)
        assert ex <= 1.0, (f"{name}: slot {int(slots[i])} (token {t}, expert {e}) off by "
                           f"{ex:.2f} x the allowance")
    say(f"  {len(pairs)} rows, {flips} elements rounded the other way at a boundary, "
        f"worst {worst:.3f} x allowance")
    free()


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_bf16", "decode_bf16", "skewed_bf16",
                                  "prefill_fp8", "prefill_bf16_shared", "prefill_mxfp4",
                                  "decode_mxfp4"])
def test_full_size_parity(name):
    cfg = CONFIGS[name]
    say("full", name)
    inp = gpu_inputs(cfg)
    # the gate of every token: logits and ids bit for bit, weights within 4 ulp
    logits, ids, w = gpu_route(cfg, inp)
    say("  oracle gate of", cfg.T, "tokens")
    ref_l, ref_ids, ref_w = oracle_route_rows(cfg, inp, np.arange(cfg.T))
    assert np.array_equal(logits.cpu().numpy(), ref_l)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert f32_ulps(w.cpu().numpy(), ref_w) <= 4
    del logits
    # the whole layer: its routing and permutation on every token
    packed = B.pack_weights(inp)
    dbg = debug_buffers(cfg)
    out = _forward(cfg, inp, dbg=dbg, packed=packed)
    assert torch.equal(dbg["topk_ids"].view(cfg.T, cfg.k), ids)
    assert torch.equal(dbg["topk_w"].view(cfg.T, cfg.k), w)
    perm = oracle.permute(ref_ids, cfg.E)
    for key, v in perm.items():
        assert np.array_equal(dbg[key].cpu().numpy(), v), key
    del dbg
    # outputs of a token sample (first and last token always)
    if cfg.T <= FULL_SAMPLE.get(name, cfg.T):
        rows = np.arange(cfg.T)
    else:
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(cfg.T, size=FULL_SAMPLE[name], replace=False))
        rows[0], rows[-1] = 0, cfg.T - 1
    say("  oracle forward of", len(rows), "tokens")
    ref, ref_rows_ids, _ = oracle_forward_rows(cfg, inp, rows)
    assert np.array_equal(ref_rows_ids, ref_ids[rows])
    sel = torch.as_tensor(rows, device="cuda")
    _outputs_ok(cfg, out[sel], ref, "native out")
    del out
    free()
    if cfg.out_dtype != F32:
        out32 = _forward(cfg, inp, out_dtype=F32, packed=packed)
        _outputs_ok(cfg, out32[sel], ref, "fp32 out")
        del out32
    del inp, packed
    free()


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_bf16_r", "decode_bf16_r",
                                  "skewed_bf16_r", "prefill_fp8_r"])
def test_stated_layout_weights_match_the_oracle(name):
    # weights passed as the workloads state them ([E][d][f], [E][f][d]) with
    # w_layout MOE_W_KN: the GEMMs read them as k-row tiles (transposing LDS
    # loads), no pack; the layer must match the oracle, and equal the packed
    # layout's output bit for bit (the same products in the same order)
    cfg = REDUCED[name]
    say("stated layout", name)
    inp = gpu_inputs(cfg)
    ref, _, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    out = forward(cfg, inp, None)
    torch.cuda.synchronize()
    _outputs_ok(cfg, out, ref, "stated layout")
    out32 = forward(cfg, inp, None, out_dtype=F32)
    packed32 = _forward(cfg, inp, out_dtype=F32)
    torch.cuda.synchronize()
    _outputs_ok(cfg, out32, ref, "stated layout, fp32 out")
    assert torch.equal(out32, packed32)


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_bf16_r", "prefill_fp8_r"])
def test_stated_layout_every_tile_height(name, block_m):
    # every k-row tile shape equals the packed layout's kernel bit for bit
    cfg = REDUCED[name]
    say("stated layout bm", name, block_m)
    inp = gpu_inputs(cfg)
    out = forward(cfg, inp, None, out_dtype=F32, block_m=block_m)
    ref = _forward(cfg, inp, out_dtype=F32, block_m=block_m)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_stated_layout_mxfp4_is_refused():
    # MXFP4 weights have no stated [K][N] form (their codes are K-major by
    # definition): MOE_ERR_UNSUPPORTED before anything is written
    cfg = REDUCED["prefill_mxfp4_r"]
    say("stated layout mxfp4")
    inp = gpu_inputs(cfg)
    p = B.problem_of(cfg, w_layout=B.MOE_W_KN)
    ws = poisoned_workspace(p)
    out = torch.full((cfg.T, cfg.d), 7.0, device="cuda").to(B.out_tensor(cfg).dtype)
    with pytest.raises(B.MoEError) as e:
        B.forward(cfg, inp, None, out=out, ws=ws)
    assert e.value.code == 2
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()


@pytest.mark.parametrize("name", ["skewed_bf16_r", "prefill_fp8_r", "prefill_mxfp4_r",
                                  "tiny_fp32"])
def test_queue_order_does_not_change_the_output(name):
    # the per-XCD queues only decide which workgroup runs which task: handing
    # each queue's tasks out in reverse or shuffled order must give the same
    # bits (every output element has exactly one writer)
    cfg = REDUCED[name]
    say("queue order", name)
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    ref = forward(cfg, inp, packed, out_dtype=F32, dbg={"queue_order": 0})
    for order in (1, 2):
        got = forward(cfg, inp, packed, out_dtype=F32, dbg={"queue_order": order})
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (name, order)


def _task_records(log, phase):
    """(index, relative start, duration, workgroup, xcd) of every record of a
    GEMM launch in a poisoned task log; times in 100 MHz ticks relative to the
    first record, unwrapped from 32 bits."""
    rec = log[phase].cpu().numpy().astype(np.int64)
    valid = (rec[:, 3] >= 0x100) & (rec[:, 3] <= 0x107)
    idx = np.nonzero(valid)[0]
    start = rec[idx, 0]
    rel = (start - start[0] + (1 << 31)) % (1 << 32) - (1 << 31)
    return idx, rel, rec[idx, 1], rec[idx, 2], rec[idx, 3] & 7


@pytest.mark.parametrize("name", ["skewed_bf16", "prefill_bf16"])
def test_task_log_every_task_once_and_queues_balanced(name):
    # per-task records of both GEMM launches of a full-size layer: every task
    # of the tile map runs exactly once, on all eight XCDs, and the
    # work-conserving queues keep the workgroups busy for most of the launch
    # even on the skewed layer, whose hottest expert holds ~15 % of the slots
    cfg = CONFIGS[name]
    say("task log", name)
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    cap = 1 << 14
    log = poisoned((2, cap, 4), torch.int32)
    dbg = {"task_log": log, "counts": poisoned(cfg.E, torch.int32)}
    out = forward(cfg, inp, packed, dbg=dbg)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().numpy()
    bm = 256  # T*k/E >= 384 on both layers
    n_mtiles = int(np.sum((counts + bm - 1) // bm))
    for phase in (0, 1):
        idx, rel, dur, wg, xcd = _task_records(log, phase)
        n = len(idx)
        assert n > 0 and n % n_mtiles == 0, (phase, n, n_mtiles)
        assert np.array_equal(idx, np.arange(n)), phase  # each task once, no other entry
        assert (dur > 0).all()
        assert set(xcd.tolist()) == set(range(8))
        span = float((rel + dur).max() - rel.min())
        busy = float(dur.sum()) / (len(np.unique(wg)) * span)
        say(f"  phase {phase + 1}: {n} tasks, {len(np.unique(wg))} workgroups, busy {busy:.3f}")
        assert busy > 0.75, (phase, busy)
    # the log is a debug output only: the layer is unchanged
    ref = forward(cfg, inp, packed)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    del inp, packed, out, ref
    free()


def test_abi_errors_launch_nothing():
    say("abi errors")
    cfg = EDGE["ragged"]
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    p = B.problem_of(cfg)
    ws = B.alloc_workspace(p)
    out = torch.full((cfg.T, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    args = dict(x=inp["x"], gate_w=inp["gate_w"], bias=None, W1t=packed["W1t"],
                W3t=packed["W3t"], W2t=packed["W2t"], W1s=None, W3s=None, W2s=None, out=out)

    def call(p_, ws_=ws, **over):
        a = dict(args)
        a.update(over)
        B.moe_forward(p_, a["x"], a["gate_w"], a["bias"], a["W1t"], a["W3t"], a["W2t"],
                      a["W1s"], a["W3s"], a["W2s"], a["out"], ws_)

    with pytest.raises(B.MoEError) as e:
        call(p, x=None)
    assert e.value.code == 1
    with pytest.raises(B.MoEError) as e:
        call(B.problem(cfg.T, cfg.d, cfg.f, cfg.E, cfg.E + 1, BF16, BF16, BF16))
    assert e.value.code == 1
    with pytest.raises(B.MoEError) as e:
        call(p, ws_=ws[:100])
    assert e.value.code == 3
    with pytest.raises(B.MoEError) as e:
        call(B.problem(cfg.T, 96, cfg.f, cfg.E, cfg.k, BF16, FP8, BF16))
    assert e.value.code in (1, 2)
    with pytest.raises(B.MoEError) as e:
        call(B.problem(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, F32, BF16, BF16))
    assert e.value.code == 1
    with pytest.raises(B.MoEError) as e:
        call(B.problem(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, BF16, BF16, BF16, 0, 9))
    assert e.value.code == 1
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()  # nothing was written


@pytest.mark.parametrize("name", ["prefill_bf16_r", "decode_bf16_r", "prefill_mxfp4_r"])
def test_forward_graph_replay(name):
    # moe_forward reads no size back to the host, so it can be captured into
    # a HIP graph; every replay (with eager work and synchronisations in
    # between) must reproduce the eager output bit for bit
    cfg = REDUCED[name]
    say("graph", name)
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    p = B.problem_of(cfg)
    ws = poisoned_workspace(p)
    out = poison_(B.out_tensor(cfg))
    ref = forward(cfg, inp, packed)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        B.forward(cfg, inp, packed, out=out, ws=ws, stream=s)  # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            B.forward(cfg, inp, packed, out=out, ws=ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, rep)
        del junk


def _random_configs(n=40, seed=1234):
    """Seeded random small layers over the supported space: dtype, E, k,
    hidden sizes (multiples of the dtype's contraction row), T, bias, shared
    experts and tile height."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wdt = [F32, BF16, FP8, MXFP4][i % 4]
        act = F32 if wdt == F32 else BF16
        m = {F32: 32, BF16: 64, FP8: 128, MXFP4: 128}[wdt]
        E = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 130]))
        k = int(rng.integers(1, min(E, 9) + 1))
        d = m * int(rng.integers(1, 5))
        f = m * int(rng.integers(1, 4))
        T = int(rng.choice([1, 5, 63, 64, 65, 200, 513]))
        cfg = MoEConfig(f"rand{i}", T, d, f, E, k, act, wdt, act, skew_bias=bool(rng.integers(0, 2)),
                        seed=i, n_shared=int(rng.choice([0, 0, 1, 2])))
        out.append((cfg, int(rng.choice([0, 16, 32, 64, 128, 256]))))
    return out


@pytest.mark.parametrize("cfg,block_m", _random_configs(), ids=lambda v: getattr(v, "name", str(v)))
def test_random_config_parity(cfg, block_m):
    say("random", cfg, block_m)
    inp = gpu_inputs(cfg)
    dbg = debug_buffers(cfg, keys=["topk_ids"])
    ref, ref_ids, _ = oracle_forward_rows(cfg, inp, np.arange(cfg.T))
    out = _forward(cfg, inp, out_dtype=F32, block_m=block_m, dbg=dbg)
    assert np.array_equal(dbg["topk_ids"].view(cfg.T, cfg.k).cpu().numpy(), ref_ids)
    _outputs_ok(cfg, out, ref, f"fp32 out bm={block_m}")
    _outputs_ok(cfg, _forward(cfg, inp, block_m=block_m), ref, "native out")
    if cfg.w_dtype != MXFP4:  # the stated weight layout gives the same bits
        kn = forward(cfg, inp, None, out_dtype=F32, block_m=block_m)
        torch.cuda.synchronize()
        assert torch.equal(kn, out)


# ---------------------------------------------------------------------------
# single-launch pipeline (moe_forward_ring): both GEMMs in one persistent
# launch with h in a bounded ring; outputs must equal moe_forward's bit for bit
# ---------------------------------------------------------------------------

RING = {
    "prefill_bf16_r": REDUCED["prefill_bf16_r"],
    "skewed_bf16_r": REDUCED["skewed_bf16_r"],
    "sh_bf16": SHARED["sh_bf16"],
    # many chunks per XCD queue, so ring slots are reused several times
    "many_chunks": MoEConfig("many_chunks", 8000, 256, 256, 64, 2, BF16, BF16, BF16),
    "one_expert": MoEConfig("one_expert", 700, 256, 128, 1, 1, BF16, BF16, BF16),
}


@pytest.mark.parametrize("name", list(RING))
def test_ring_forward_equals_forward(name):
    cfg = RING[name]
    say("ring", name)
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    for out_dtype in (F32, BF16):
        ref = forward(cfg, inp, packed, out_dtype=out_dtype, block_m=256)
        for rep in range(2):
            got = forward_ring(cfg, inp, packed, out_dtype=out_dtype, block_m=256)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (name, out_dtype, rep)
    ref64, _, _ = oracle_forward_rows(cfg, inp, np.arange(min(cfg.T, 64)))
    out = forward_ring(cfg, inp, packed, out_dtype=F32, block_m=256)
    torch.cuda.synchronize()
    _outputs_ok(cfg, out[: ref64.shape[0]], ref64, "ring vs oracle")


@pytest.mark.parametrize("name", ["prefill_bf16", "skewed_bf16", "prefill_bf16_shared"])
def test_ring_full_size_equals_forward(name):
    cfg = CONFIGS[name]
    say("ring full", name)
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    ref = forward(cfg, inp, packed)
    got = forward_ring(cfg, inp, packed)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), name
    del inp, packed, ref, got
    free()


def test_ring_unsupported_shapes_launch_nothing():
    for name in ("decode_bf16", "prefill_fp8_r", "tiny_fp32"):
        cfg = CONFIGS.get(name) or REDUCED[name]
        p = B.problem_of(cfg, T=min(cfg.T, 64))
        with pytest.raises(B.MoEError, match="UNSUPPORTED"):
            B.ring_workspace_size(p)


def test_ring_graph_replay():
    cfg = RING["many_chunks"]
    say("ring graph")
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    p = B.problem_of(cfg, block_m=256)
    ws = poisoned(B.ring_workspace_size(p), torch.uint8)
    out = B.out_tensor(cfg)
    ref = forward(cfg, inp, packed, block_m=256)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        forward_ring(cfg, inp, packed, out=out, ws=ws, block_m=256, stream=s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            forward_ring(cfg, inp, packed, out=out, ws=ws, block_m=256, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        del junk


def test_ring_repeated_runs_identical():
    # the ring's counters order every h handoff: thirty back-to-back runs of
    # the full-size skewed layer (hot expert: the longest chunk chains, most
    # stealing) must each reproduce moe_forward bit for bit
    cfg = CONFIGS["skewed_bf16"]
    say("ring repeated", cfg.name)
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    ref = forward(cfg, inp, packed)
    p = B.problem_of(cfg)
    ws = poisoned(B.ring_workspace_size(p), torch.uint8)
    outs = [forward_ring(cfg, inp, packed, ws=ws) for _ in range(30)]
    torch.cuda.synchronize()
    assert not B.ring_failed(p, ws)
    for i, o in enumerate(outs):
        assert torch.equal(o, ref), i
    del inp, packed, ref, outs
    free()


def test_ring_error_flag_reports_a_wait_that_gave_up():
    # the failure report of the bounded waits, forced from the host: with
    # every target out of reach each wait gives up after 4 polls, the launch
    # still drains its queues, and the flag reads 1; the next call on the same
    # workspace clears it and is correct again
    cfg = RING["many_chunks"]
    say("ring error flag")
    inp = gpu_inputs(cfg)
    packed = B.pack_weights(inp)
    p = B.problem_of(cfg, block_m=256)
    ws = poisoned(B.ring_workspace_size(p), torch.uint8)
    ref = forward(cfg, inp, packed, block_m=256)
    out = forward_ring(cfg, inp, packed, ws=ws, block_m=256)
    assert not B.ring_failed(p, ws)
    assert torch.equal(out, ref)
    forward_ring(cfg, inp, packed, ws=ws, block_m=256,
              dbg={"ring_poll_limit": 4, "ring_force_timeout": 1})
    assert B.ring_failed(p, ws)
    out = forward_ring(cfg, inp, packed, ws=ws, block_m=256)
    assert not B.ring_failed(p, ws)
    assert torch.equal(out, ref)
    # a poll limit alone only bounds the waits: a generous one changes nothing
    out = forward_ring(cfg, inp, packed, ws=ws, block_m=256,
                    dbg={"ring_poll_limit": 1 << 20})
    assert not B.ring_failed(p, ws)
    assert torch.equal(out, ref)


def test_ring_concurrent_on_two_streams():
    # every wait of the ring targets tasks pulled earlier from the same queue,
    # so it needs no co-residency: two ring launches (own workspaces) on two
    # streams, each sharing the GPU with the other, still match moe_forward
    cfgs = [RING["many_chunks"], RING["prefill_bf16_r"]]
    say("ring two streams", [c.name for c in cfgs])
    inps = [gpu_inputs(c) for c in cfgs]
    packs = [B.pack_weights(i) for i in inps]
    ref = [forward(c, i, p, block_m=256) for c, i, p in zip(cfgs, inps, packs)]
    probs = [B.problem_of(c, block_m=256) for c in cfgs]
    wss = [poisoned(B.ring_workspace_size(p), torch.uint8) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for rep in range(3):
        for j in (0, 1):
            with torch.cuda.stream(streams[j]):
                outs[j].append(forward_ring(cfgs[j], inps[j], packs[j], ws=wss[j], block_m=256,
                                         stream=streams[j]))
    torch.cuda.synchronize()
    for j in (0, 1):
        assert not B.ring_failed(probs[j], wss[j])
        for o in outs[j]:
            assert torch.equal(o, ref[j]), cfgs[j].name
