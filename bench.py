#!/usr/bin/env python
"""Benchmark of the one-GPU MoE layer forward on MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one whole-layer moe_forward (gate, FP8 quantisation of x when
the layer is FP8, histogram/scan/scatter, W1/W3 + SwiGLU GEMM, W2 GEMM,
combine) on inputs already resident in HBM, weights packed once before the
timed region.  Prints ONE JSON line: tokens/s of the whole layer, the
roofline of the dominant kernel timed live with HIP events recorded inside
the call, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# dense MFMA peaks: fp32, bf16, fp8; FP4 weights x FP8 activations run at the
# fp8 rate (the scaled MFMA with one FP8 operand), so MXFP4 layers use it too
PEAK_TFLOPS = {0: 157.3, 1: 2516.6, 2: 5033.2, 3: 5033.2}
PEAK_HBM_GBPS = 8000.0
STAGES = ["gate", "quant_x", "permute", "gemm_w13_swiglu", "gemm_w2", "combine"]


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _device_info():
    """CU count and maximum shader clock as rocminfo reports them for the GPU
    agent, and the dense peaks they imply (per CU and clock: 4096 bf16, 8192
    fp8 and 256 fp32 MFMA FLOP)."""
    import subprocess
    cus = mhz = None
    name = None
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        agent = {}
        for line in txt.splitlines() + ["Agent end"]:
            line = line.strip()
            if line.startswith("Agent ") or line.startswith("*******"):
                if agent.get("Device Type") == "GPU" and cus is None:
                    name = agent.get("Name")
                    cus = int(agent["Compute Unit"]) if "Compute Unit" in agent else None
                    mhz = (int(agent["Max Clock Freq. (MHz)"])
                           if "Max Clock Freq. (MHz)" in agent else None)
                agent = {}
            elif ":" in line:
                k, v = line.split(":", 1)
                agent.setdefault(k.strip(), v.strip())
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    info = {"agent": name, "cus": cus, "max_clock_mhz": mhz}
    if cus and mhz:
        f = cus * mhz * 1e6
        info["derived_peak_tflops"] = {"bf16": f * 4096 / 1e12, "fp8": f * 8192 / 1e12,
                                       "fp32_mfma": f * 256 / 1e12}
    return info


def _copy_gbps(torch):
    """Device-to-device copy of 1 GiB (read + write bytes per second)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(3):
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2.0 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a, b
    return best


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _events(hip, n):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    return evs


def _elapsed(hip, a, b):
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return ms.value


def _src_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "mixture_experts_layer_softmax_amd", "csrc"))):
        with open(os.path.join(ROOT, "mixture_experts_layer_softmax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, kernel):
    """HBM bytes per launch from a committed rocprofv3 counter summary, valid
    only while the kernel sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("src_hash") != _src_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _stage_work(cfg, counts):
    """Algorithmic work per launch of each GEMM stage: FLOPs, and HBM bytes
    (weights of the experts that receive a token, activations in, outputs).
    Shared experts count as experts hit by every token: T more rows each."""
    import numpy as np
    # bytes per weight / activation / h element; MXFP4: half-byte codes and
    # MX FP8 activations, each with one E8M0 byte per 32 elements
    es = {0: 4, 1: 2, 2: 1, 3: 0.5 + 1 / 32}[cfg.w_dtype]
    ae = {0: 4, 1: 2}[cfg.act_dtype] if cfg.w_dtype < 2 else (1 if cfg.w_dtype == 2 else 1 + 1 / 32)
    he = {0: 4, 1: 2, 2: 1, 3: 1 + 1 / 32}[cfg.w_dtype]
    hit = int(np.count_nonzero(counts)) + cfg.n_shared
    n = cfg.T * (cfg.k + cfg.n_shared)
    w13 = dict(flops=4.0 * n * cfg.d * cfg.f,
               bytes=hit * 2.0 * cfg.d * cfg.f * es + cfg.T * cfg.d * ae + n * cfg.f * he)
    w2 = dict(flops=2.0 * n * cfg.d * cfg.f,
              bytes=hit * 1.0 * cfg.d * cfg.f * es + n * cfg.f * he + n * cfg.d * 4.0)
    return {"gemm_w13_swiglu": w13, "gemm_w2": w2, "hit_experts": hit}


def _cpu_baseline(cfg, inp, out_gpu, target_s):
    """The CPU oracle as it stands, timed on a bounded token sample."""
    import numpy as np
    import torch

    import oracle
    from mixture_experts_layer_softmax_amd.inputs import host_arrays, host_weight

    orc = {0: oracle.ORC_F32, 1: oracle.ORC_BF16, 2: oracle.ORC_FP8, 3: oracle.ORC_MXFP4}
    gw = host_arrays(inp["gate_w"])
    bias = None if inp.get("bias") is None else inp["bias"].cpu().numpy()
    host_w = {}

    def run(rows):
        x = host_arrays(inp["x"][torch.as_tensor(rows, device=inp["x"].device)])
        _, ids, _ = oracle.route(x, gw, bias, cfg.k, orc[cfg.act_dtype])
        need = set(int(v) for v in ids.reshape(-1)) | set(range(cfg.E, cfg.E + cfg.n_shared))
        for e in sorted(need):
            if e not in host_w:
                host_w[e] = {}
                for n in ("W1", "W3", "W2"):
                    host_w[e][n], host_w[e][n + "s"] = host_weight(cfg, inp, n, e)
        W = {n: [host_w.get(e, {}).get(n) for e in range(cfg.E + cfg.n_shared)]
             for n in ("W1", "W3", "W2", "W1s", "W3s", "W2s")}
        sc = cfg.w_dtype in (2, 3)
        t0 = time.perf_counter()
        out, _, _ = oracle.forward(x, gw, bias, W["W1"], W["W3"], W["W2"], cfg.k,
                                   orc[cfg.act_dtype], orc[cfg.w_dtype],
                                   W1s=W["W1s"] if sc else None,
                                   W3s=W["W3s"] if sc else None,
                                   W2s=W["W2s"] if sc else None, n_shared=cfg.n_shared)
        return out, time.perf_counter() - t0

    rng = np.random.default_rng(0)
    n0 = min(cfg.T, 8)
    rows0 = np.sort(rng.choice(cfg.T, size=n0, replace=False))
    _, t_probe = run(rows0)
    n = int(min(cfg.T, max(n0, n0 * target_s / max(t_probe, 1e-3))))
    rows = np.sort(rng.choice(cfg.T, size=n, replace=False))
    ref, secs = run(rows)
    got = out_gpu[torch.as_tensor(rows, device=out_gpu.device)].double().cpu().numpy()
    rms = math.sqrt(float(np.mean(ref ** 2))) or 1.0
    diff = np.abs(got - ref)
    err = {"max_abs_err_over_rms": float(diff.max()) / rms}
    if out_gpu.dtype == torch.bfloat16:
        # rounding the exact result to bf16 alone costs up to half a bf16 ulp
        half_ulp = 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        err["max_excess_over_half_bf16_ulp_over_rms"] = float(np.maximum(diff - half_ulp, 0).max()) / rms
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    return {"value": n / secs, "unit": "tokens/s", "cores": cores, "cpu": _cpu_model(),
            "kind": "oracle",
            "sample": f"{n} of {cfg.T} tokens (seeded random rows), full layer forward per "
                      f"token, {secs:.1f} s", "seconds": secs}, err


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 50 warm-up steps: the shader clock ramps up over the first ~50 ms of
    # load (prefill_bf16 GEMMs at ~2.08 GHz after 5 steps, ~2.23 GHz after 50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-m", type=int, default=0, help="expert tile height (0 = auto)")
    ap.add_argument("--ring", action="store_true",
                    help="time moe_forward_ring (both GEMMs in one launch, h in a bounded ring)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_softmax_amd import binding as B
    from mixture_experts_layer_softmax_amd.configs import CONFIGS
    from mixture_experts_layer_softmax_amd.inputs import make_inputs

    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    B.load()
    inp = make_inputs(cfg, device="cuda")
    packed = B.pack_weights(inp)
    p = B.problem_of(cfg, block_m=args.block_m)
    if args.ring:
        ws = torch.empty(B.ring_workspace_size(p), dtype=torch.uint8, device="cuda")
    else:
        ws = B.alloc_workspace(p)
    out = B.out_tensor(cfg)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    hip = _hip()
    nev = B.NUM_STAGE_EVENTS
    evs = [_events(hip, nev) for _ in range(args.steps)]

    def step(dbg=None):
        if args.ring:
            B.moe_forward_ring(p, inp["x"], inp["gate_w"], inp.get("bias"), packed["W1t"],
                               packed["W3t"], packed["W2t"], out, ws, dbg=dbg, stream=stream)
            return
        B.moe_forward(p, inp["x"], inp["gate_w"], inp.get("bias"), packed["W1t"],
                      packed["W3t"], packed["W2t"], packed.get("W1s"), packed.get("W3s"),
                      packed.get("W2s"), out, ws, dbg=dbg, stream=stream)

    for _ in range(args.warmup):
        step({"counts": counts})
    torch.cuda.synchronize()

    # Timed steps: HIP events only around the two GEMM launches (stage
    # boundaries 3, 4, 5), on the stream moe_forward launches on -- every
    # event record costs the GPU a few microseconds, so the full per-stage
    # breakdown comes from a separate, untimed pass below.
    t0 = time.perf_counter()
    clock = torch.zeros(4, dtype=torch.int64, device="cuda")
    gemm_only = (3, 4, 5)
    for i in range(args.steps):
        sel = [evs[i][j] if j in gemm_only else None for j in range(nev)]
        step({"stage_events": sel, "gemm_clock": clock})
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed_gemm_ms = {
        "gemm_w13_swiglu": float(np.mean([_elapsed(hip, e[3], e[4]) for e in evs])),
        "gemm_w2": float(np.mean([_elapsed(hip, e[4], e[5]) for e in evs])),
    }
    ck = clock.cpu().numpy().astype(np.float64)
    sustained = {name: (1e2 * ck[2 * i] / ck[2 * i + 1] if ck[2 * i + 1] > 0 else None)
                 for i, name in enumerate(("gemm_w13_swiglu", "gemm_w2"))}
    if args.ring:
        sustained = None

    # per-stage breakdown (untimed): every stage boundary recorded
    nbreak = min(args.steps, 10)
    for i in range(nbreak):
        step({"stage_events": evs[i]})
    torch.cuda.synchronize()
    stage_ms = {}
    for s, name in enumerate(STAGES, start=1):
        stage_ms[name] = float(np.mean([_elapsed(hip, e[s - 1], e[s]) for e in evs[:nbreak]]))
    gpu_ms = _elapsed(hip, evs[0][0], evs[nbreak - 1][-1]) / nbreak
    per_step = np.array([_elapsed(hip, e[0], e[-1]) for e in evs[:nbreak]])
    step_stats = {"median": float(np.median(per_step)), "min": float(per_step.min()),
                  "p90": float(np.percentile(per_step, 90))}
    for e in evs:
        for v in e:
            hip.hipEventDestroy(v)

    ms_per_step = elapsed * 1e3 / args.steps
    value = cfg.T * args.steps / elapsed
    work = _stage_work(cfg, counts.cpu().numpy())
    if args.ring:
        # one launch runs both GEMMs: its time is stage 4, stage 5 is empty
        stage_ms["gemm_ring"] = stage_ms.pop("gemm_w13_swiglu") + stage_ms.pop("gemm_w2")
        timed_gemm_ms = {"gemm_ring": timed_gemm_ms["gemm_w13_swiglu"]
                         + timed_gemm_ms["gemm_w2"]}
        work["gemm_ring"] = {k: work["gemm_w13_swiglu"][k] + work["gemm_w2"][k]
                             for k in ("flops", "bytes")}
        dom = "gemm_ring"
    else:
        dom = max(("gemm_w13_swiglu", "gemm_w2"), key=lambda k: timed_gemm_ms[k])
    dom_s = timed_gemm_ms[dom] * 1e-3
    decode = cfg.T * cfg.k / cfg.E < 16  # expected rows per routed expert
    copy_gbps = _copy_gbps(torch)
    if decode:
        achieved = work[dom]["bytes"] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS, "frac_of_measured_copy": achieved / copy_gbps}
    else:
        achieved = work[dom]["flops"] / dom_s / 1e12
        peak = PEAK_TFLOPS[cfg.w_dtype]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    roof["kernel"] = dom
    roof["avg_launch_us"] = dom_s * 1e6  # HIP events around each launch of the timed loop
    roof["traffic"] = _traffic(cfg.name, dom)
    layer_flops = cfg.expert_flops
    layer = {
        "expert_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "mfma_frac_of_peak": layer_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_TFLOPS[cfg.w_dtype],
        "alg_hbm_GBps": (work["gemm_w13_swiglu"]["bytes"] + work["gemm_w2"]["bytes"])
        / (ms_per_step * 1e-3) / 1e9,
        "hit_experts": work["hit_experts"],
        "gpu_event_ms_per_step": gpu_ms,
        "gpu_event_ms_per_step_stats": step_stats,
    }
    device = _device_info()
    device["sustained_clock_mhz"] = sustained
    device["measured_copy_GBps"] = copy_gbps

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = _cpu_baseline(cfg, inp, out, args.cpu_seconds)

    dtype = {0: "f32", 1: "bf16", 2: "fp8e4m3", 3: "mxfp4xmxfp8"}[cfg.w_dtype]
    line = {
        "metric": "MoE-layer tokens/s on 1 MI355X; MFMA % peak (prefill), HBM GB/s (decode)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f, "E": cfg.E,
                   "top_k": cfg.k, "n_shared": cfg.n_shared, "parallelism": "single GPU",
                   "gemms": "one launch, h ring" if args.ring else "two launches"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages_ms": stage_ms,
        "layer": layer,
        "device": device,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
