"""Seeded synthetic inputs shared by the GPU path and the CPU oracle.

This module only draws random tensors and stores them in the layer's input
formats; it holds none of the layer's own arithmetic.  Both sides consume the
exact bits produced here.

Recipe (per workload, seed s):
  x       ~ N(0, 1)     [T x d], rounded once to the activation type
  gate_w  ~ N(0, 0.02)  [d x E] (0.02 is the standard deviation)
  W1, W3  ~ N(0, 0.02)  [E+S][d][f];  W2 ~ N(0, 0.02) [E+S][f][d] (S shared
          experts drawn after the E routed ones)
  bias (skewed workload): bias_e = -1.2 ln(pi(e) + 1), pi a seeded random
          permutation of the experts, fp32
  FP8 weights: drawn fp32, then stored as E4M3FN codes with one fp32 scale per
          128x128 (K, N) block (scale = block amax / 448, codes = the value /
          scale cast by torch's float8_e4m3fn conversion after a clamp to
          +-448).  These codes and scales *are* the weights.
  MXFP4 weights: drawn fp32, then stored in OCP MX FP4: per column n and
          block of 32 consecutive K elements, X = floor(log2(amax)) - 2 (0 for
          an all-zero block, clamped to [-127, 127]), the E8M0 byte X + 127
          and E2M1 codes of v * 2^-X rounded to nearest even (saturating at
          6), packed K-major [E][N][K/2] (element 2i in the low nibble of byte
          i) with scales [E][N][K/32].  These codes and scales are the
          weights.
Every tensor has its own torch.Generator seeded from (seed, tensor id), so
the draw order does not matter.  Draws on a CUDA device use that device's
generator, draws on the CPU the CPU one: the bits differ between the two, so
a comparison always copies the one set of bits to the other side.
"""
from __future__ import annotations

import torch

from .configs import BF16, F32, FP8, MXFP4, MoEConfig

_IDS = {"x": 1, "gate_w": 2, "W1": 3, "W3": 4, "W2": 5, "perm": 6}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + _IDS[name])
    return g


def _tdtype(code: int):
    return {F32: torch.float32, BF16: torch.bfloat16}[code]


def _normal(shape, std, g, device):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def skew_bias(E: int, seed: int) -> torch.Tensor:
    """bias_e = -1.2 ln(pi(e)+1) for a seeded random permutation pi (CPU)."""
    pi = torch.randperm(E, generator=_gen(seed, "perm", "cpu"))
    b = -1.2 * torch.log(pi.to(torch.float64) + 1.0)
    return b.to(torch.float32)


def fp8_block_quantize(w: torch.Tensor):
    """Store an fp32 [K x N] matrix as E4M3FN codes (uint8) + fp32 scales
    [ceil(K/128) x ceil(N/128)], one scale per 128x128 block."""
    K, N = w.shape
    kb, nb = (K + 127) // 128, (N + 127) // 128
    pad = torch.zeros((kb * 128, nb * 128), dtype=torch.float32, device=w.device)
    pad[:K, :N] = w
    blocks = pad.view(kb, 128, nb, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).clamp_(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(kb * 128, nb * 128)[:K, :N]
    return codes.contiguous(), scale.contiguous()


# code of each E2M1 magnitude m, indexed by 2*m (0, .5, 1, 1.5, 2, 3, 4, 6)
_E2M1_CODE = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4, 6: 5, 8: 6, 12: 7}


def mxfp4_quantize(w: torch.Tensor):
    """Store an fp32 [K x N] matrix (K a multiple of 32) as OCP MX FP4:
    packed codes [N x K/2] uint8 and E8M0 scales [N x K/32] uint8."""
    K, N = w.shape
    wt = w.t().contiguous().view(N, K // 32, 32).to(torch.float64)
    amax = wt.abs().amax(dim=-1)
    _, e = torch.frexp(amax)  # amax = m * 2^e, 0.5 <= m < 1
    x = torch.where(amax > 0, (e.to(torch.int64) - 1 - 2).clamp(-127, 127),
                    torch.zeros_like(e, dtype=torch.int64))
    a = wt.abs() * torch.pow(2.0, -x.to(torch.float64))[..., None]  # exact
    quantum = torch.where(a < 2, 0.5, torch.where(a < 4, 1.0, 2.0))
    r = (torch.round(a / quantum) * quantum).clamp(max=6.0)  # round half to even
    lut = torch.zeros(13, dtype=torch.uint8, device=w.device)
    for m2, c in _E2M1_CODE.items():
        lut[m2] = c
    code = lut[(r * 2).to(torch.int64)] | (torch.signbit(wt).to(torch.uint8) << 3)
    code = code.view(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, (x + 127).to(torch.uint8).contiguous()


def unpack_mxfp4(packed: torch.Tensor) -> torch.Tensor:
    """[.., N, K/2] packed codes -> [.., N, K] one code per byte."""
    lo, hi = packed & 15, packed >> 4
    return torch.stack([lo, hi], dim=-1).flatten(-2)


def make_inputs(cfg: MoEConfig, device="cpu", seed: int | None = None,
                experts=None, progress=None) -> dict:
    """Draw the layer inputs of `cfg` on `device`.

    Returns a dict with x, gate_w, bias (or None), W1, W3, W2 and, for FP8
    weights, W1s, W3s, W2s.  Weight tensors are [E+S][K][N] in the stated
    layouts (W1/W3 [.][d][f], W2 [.][f][d]), the S shared experts last; MXFP4
    weights are the packed K-major codes [.][N][K/2] and W1s/W3s/W2s their
    E8M0 scales [.][N][K/32].
    `experts` (optional) limits the weight draw to those expert indices
    (others stay zero) -- a test
    convenience only; the draws of the listed experts do not change.
    `progress` (optional) is called as progress(name, experts_drawn, NE)
    after every 64 experts of each weight matrix.
    """
    seed = cfg.seed if seed is None else seed
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    NE = E + cfg.n_shared  # weight sets: routed, then shared
    act = _tdtype(cfg.act_dtype)
    out = {}
    out["x"] = _normal((T, d), 1.0, _gen(seed, "x", device), device).to(act)
    out["gate_w"] = _normal((d, E), 0.02, _gen(seed, "gate_w", device), device).to(act)
    out["bias"] = skew_bias(E, seed).to(device) if cfg.skew_bias else None

    wanted = set(range(NE)) if experts is None else set(int(e) for e in experts)
    for name, (K, N) in (("W1", (d, f)), ("W3", (d, f)), ("W2", (f, d))):
        g = _gen(seed, name, device)
        if cfg.w_dtype == MXFP4:
            codes = torch.zeros((NE, N, K // 2), dtype=torch.uint8, device=device)
            scales = torch.zeros((NE, N, K // 32), dtype=torch.uint8, device=device)
        elif cfg.w_dtype == FP8:
            codes = torch.zeros((NE, K, N), dtype=torch.uint8, device=device)
            scales = torch.zeros((NE, (K + 127) // 128, (N + 127) // 128),
                                 dtype=torch.float32, device=device)
        else:
            codes = torch.zeros((NE, K, N), dtype=_tdtype(cfg.w_dtype), device=device)
            scales = None
        for e in range(NE):
            # every expert is drawn in order so that a subset draw reproduces
            # the full draw bit for bit
            w = _normal((K, N), 0.02, g, device)
            if progress is not None and ((e + 1) % 64 == 0 or e + 1 == NE):
                progress(name, e + 1, NE)
            if e not in wanted:
                continue
            if cfg.w_dtype == MXFP4:
                c, s = mxfp4_quantize(w)
                codes[e] = c
                scales[e] = s
            elif cfg.w_dtype == FP8:
                c, s = fp8_block_quantize(w)
                codes[e] = c
                scales[e] = s
            else:
                codes[e] = w.to(codes.dtype)
        out[name] = codes
        if scales is not None:
            out[name + "s"] = scales
    return out


def expected_tokens_per_expert(cfg: MoEConfig) -> float:
    return cfg.T * cfg.k / cfg.E


def bf16_bits(t: torch.Tensor):
    """Raw uint16 bit patterns of a bf16 tensor as a numpy array (CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def host_arrays(t: torch.Tensor):
    """numpy view of a tensor in the oracle's storage convention: fp32 as
    float32, bf16 as uint16 bits, FP8 codes as uint8."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def host_weight(cfg: MoEConfig, inp: dict, name: str, e: int):
    """Expert e's weight `name` (W1, W3, W2) in host memory as a [K x N] array
    in the storage convention of host_arrays, with its scales (FP8: fp32
    [K/128 x N/128]; MXFP4: E8M0 bytes [K/32 x N]; otherwise None).  MXFP4
    codes are unpacked from the K-major nibble layout to one code per byte:
    a change of layout only, the bits are the ones the GPU reads."""
    if cfg.w_dtype == MXFP4:
        codes = unpack_mxfp4(inp[name][e]).t().contiguous().cpu().numpy()
        return codes, inp[name + "s"][e].t().contiguous().cpu().numpy()
    if cfg.w_dtype == FP8:
        return host_arrays(inp[name][e]), inp[name + "s"][e].cpu().numpy()
    return host_arrays(inp[name][e]), None


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

