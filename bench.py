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
# stage name -> the pair of moe_debug stage events around it (event 1, between
# the gate and its activation quantisation, is not recorded: the quantisation
# runs inside the gate kernel, and an event there only adds its own cost)
STAGES = {"gate": (0, 2), "permute": (2, 3), "gemm_w13_swiglu": (3, 4), "gemm_w2": (4, 5),
          "combine": (5, 6)}


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
    """Hash of the sources the grouped-GEMM kernels are built from: counter
    figures taken on them stay valid until one of these files changes."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "launch.hpp", "device_common.hpp"):
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
    # Y: fp32 on fp32 layers, bf16 on MXFP4 layers, else fp16 codes with one
    # exponent byte per 32 columns
    ye = {0: 4.0, 1: 2.0 + 1 / 32, 2: 2.0 + 1 / 32, 3: 2.0}[cfg.w_dtype]
    w2 = dict(flops=2.0 * n * cfg.d * cfg.f,
              bytes=hit * 1.0 * cfg.d * cfg.f * es + n * cfg.f * he + n * cfg.d * ye)
    return {"gemm_w13_swiglu": w13, "gemm_w2": w2, "hit_experts": hit}


def _cpu_baseline(cfg, inp, out_gpu, out32_gpu, target_s):
    """The CPU oracle as it stands, timed on a bounded token sample; the same
    sample checks the run's outputs (the workload's own output type, and the
    fp32-output run when there is one)."""
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
    if secs < 0.5 * target_s and n < cfg.T:
        # the probe overstates the per-token cost when each expert's fixed
        # cost dominates a few tokens: size the sample again from this run
        n = int(min(cfg.T, n * target_s / max(secs, 1e-3)))
        rows = np.sort(rng.choice(cfg.T, size=n, replace=False))
        ref, secs = run(rows)
    sel = torch.as_tensor(rows, device=out_gpu.device)
    got = out_gpu[sel].double().cpu().numpy()
    rms = math.sqrt(float(np.mean(ref ** 2))) or 1.0
    diff = np.abs(got - ref)
    err = {"tokens": int(n), "max_abs_err_over_rms": float(diff.max()) / rms}
    if out_gpu.dtype == torch.bfloat16:
        # rounding the exact result to bf16 alone costs up to half a bf16 ulp
        half_ulp = 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        err["max_excess_over_half_bf16_ulp_over_rms"] = float(np.maximum(diff - half_ulp, 0).max()) / rms
    if out32_gpu is not None:
        got32 = out32_gpu[sel].double().cpu().numpy()
        err["fp32_out_max_abs_err_over_rms"] = float(np.abs(got32 - ref).max()) / rms
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    return {"value": n / secs, "unit": "tokens/s", "cores": cores, "cpu": _cpu_model(),
            "kind": "oracle",
            "sample": f"{n} of {cfg.T} tokens (seeded random rows), full layer forward per "
                      f"token, {secs:.1f} s", "seconds": secs}, err


def _kernel_short_name(name):
    """'void moe::(anonymous namespace)::gemm<1, 2>(moe::GemmArgs)' ->
    'gemm<1, 2>': return type, namespaces and the parameter list dropped."""
    import re
    name = re.sub(r"^void ", "", name.strip())
    name = re.sub(r"^moe::\(anonymous namespace\)::", "", name)
    depth = 0
    for i, ch in enumerate(name):  # cut at the '(' of the parameter list
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i].strip()
    return name


def trace_summary(csv_path, warmup, steps, workloads):
    """Markdown summary of a rocprofv3 kernel trace (--kernel-trace, csv) of a
    bench.py run: per workload, per library kernel, the dispatch count, the
    average over every dispatch and the average over the timed steps alone.
    Each moe_forward call starts with exactly one gate_kernel dispatch, so
    the library's dispatches (in start order) split into forward calls; the
    workloads ran one after another in the given order, each with `warmup`
    untimed calls first and `steps` timed ones next (then untimed ones)."""
    import csv
    import re
    lib = re.compile(r"^(gate_kernel|topk_kernel|hist_kernel|scan_kernel|scatter_kernel|"
                     r"permute_one_kernel|quant_fp8_kernel|quant_mx_kernel|"
                     r"grouped_gemm_kernel|ring_gemm_kernel|combine_kernel|zero_kernel)")
    rows = []
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            short = _kernel_short_name(r["Kernel_Name"])
            if lib.match(short):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short))
    rows.sort()
    calls = []  # forward calls: lists of (kernel, microseconds)
    for t0, t1, name in rows:
        if name.startswith("gate_kernel") or not calls:
            calls.append([])
        calls[-1].append((name, (t1 - t0) / 1e3))
    # a workload's calls: consecutive calls whose gate kernel has the same name
    groups = []
    for c in calls:
        if not groups or groups[-1][0] != c[0][0]:
            groups.append((c[0][0], []))
        groups[-1][1].append(c)
    out = []
    for (gate, cs), wl in zip(groups, workloads):
        out.append(f"\n### {wl} ({len(cs)} forward calls; timed: calls {warmup + 1}.."
                   f"{warmup + steps})\n")
        out.append("| kernel | calls | avg us | timed steps avg us | % of timed layer |")
        out.append("|---|---|---|---|---|")
        per = {}
        for i, c in enumerate(cs):
            for name, us in c:
                d = per.setdefault(name, [[], []])
                d[0].append(us)
                if warmup <= i < warmup + steps:
                    d[1].append(us)
        tot = sum(sum(v[1]) for v in per.values()) or 1.0
        for name, (a, tm) in sorted(per.items(), key=lambda kv: -sum(kv[1][1])):
            avg_t = f"{sum(tm) / len(tm):.1f}" if tm else "-"
            out.append(f"| {name} | {len(a)} | {sum(a) / len(a):.1f} | {avg_t} | "
                       f"{100.0 * sum(tm) / tot:.1f} |")
    return "\n".join(out)


def counter_summary(csv_path):
    """Markdown table of a rocprofv3 --pmc run (csv): per kernel, grid size
    and counter, the number of dispatches and the mean value per dispatch
    (the grid size tells apart dispatches of one kernel on different sizes,
    such as the runtime's copy kernel on the 1 GiB calibration copy)."""
    import csv
    acc = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            name = _kernel_short_name(r["Kernel_Name"])
            if name.startswith("at::native"):
                continue
            key = (name, int(r.get("Grid_Size") or 0), r["Counter_Name"])
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
    out = ["| kernel | grid | counter | dispatches | mean per dispatch |",
           "|---|---|---|---|---|"]
    for (name, grid, ctr), v in sorted(acc.items()):
        out.append(f"| {name[:90]} | {grid} | {ctr} | {len(v)} | {sum(v) / len(v):.1f} |")
    return "\n".join(out)


def _free(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def measure(cfg, args, steps, warmup, cpu_seconds, hip, copy_gbps):
    """Time `steps` whole-layer forwards of cfg after `warmup` untimed ones.
    Returns the per-workload record (tokens/s, roofline of the dominant GEMM
    launch, stage breakdown) and a function that later adds the CPU-oracle
    baseline and parity sample to it (it launches no kernel of the library;
    it copies the rows it needs to the host) and frees the workload's device
    memory: the GPU phases of several workloads can then run back to back,
    with no host-only stretch between them."""
    import numpy as np
    import torch

    from mixture_experts_layer_softmax_amd import binding as B
    from mixture_experts_layer_softmax_amd.inputs import make_inputs

    _say(f"{cfg.name}: drawing inputs")
    # (a line per 64 experts: under a counter-collecting profiler the draw
    # of a 256-expert layer runs for minutes)
    inp = make_inputs(cfg, device="cuda",
                      progress=lambda n, i, ne: _say(f"{cfg.name}: {n} {i}/{ne} experts drawn"))
    t_pack = time.perf_counter()
    if args.stated_weights:  # the layouts the workload states, read without a pack
        packed = {"W1t": inp["W1"], "W3t": inp["W3"], "W2t": inp["W2"]}
        packed.update({k: inp[k] for k in ("W1s", "W3s", "W2s") if k in inp})
        layout = B.MOE_W_KN
    else:
        packed = B.pack_weights(inp)
        layout = B.MOE_W_NK
    torch.cuda.synchronize()
    pack_s = time.perf_counter() - t_pack
    p = B.problem_of(cfg, block_m=args.block_m, w_layout=layout)
    if args.ring:
        ws = torch.empty(B.ring_workspace_size(p), dtype=torch.uint8, device="cuda")
    else:
        ws = B.alloc_workspace(p)
    out = B.out_tensor(cfg)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    nev = B.NUM_STAGE_EVENTS
    evs = [_events(hip, nev) for _ in range(steps)]

    def step(dbg=None, o=out, pp=p):
        if args.ring:
            B.moe_forward_ring(pp, inp["x"], inp["gate_w"], inp.get("bias"), packed["W1t"],
                               packed["W3t"], packed["W2t"], o, ws, dbg=dbg, stream=stream)
            return
        B.moe_forward(pp, inp["x"], inp["gate_w"], inp.get("bias"), packed["W1t"],
                      packed["W3t"], packed["W2t"], packed.get("W1s"), packed.get("W3s"),
                      packed.get("W2s"), o, ws, dbg=dbg, stream=stream)

    for _ in range(warmup):
        step({"counts": counts})
    torch.cuda.synchronize()

    # Timed steps: HIP events only around the two GEMM launches (stage
    # boundaries 3, 4, 5), on the stream moe_forward launches on -- every
    # event record costs the GPU a few microseconds, so the full per-stage
    # breakdown comes from a separate, untimed pass below.
    _say(f"{cfg.name}: {warmup} warm-up steps done, timing {steps}")
    t0 = time.perf_counter()
    clock = torch.zeros(4, dtype=torch.int64, device="cuda")
    gemm_only = (3, 4, 5)
    for i in range(steps):
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
    nbreak = min(steps, 10)
    for i in range(nbreak):
        step({"stage_events": [None if j == 1 else v for j, v in enumerate(evs[i])]})
    torch.cuda.synchronize()
    stage_ms = {}
    for name, (a, b) in STAGES.items():
        stage_ms[name] = float(np.mean([_elapsed(hip, e[a], e[b]) for e in evs[:nbreak]]))
    gpu_ms = _elapsed(hip, evs[0][0], evs[nbreak - 1][-1]) / nbreak
    per_step = np.array([_elapsed(hip, e[0], e[-1]) for e in evs[:nbreak]])
    step_stats = {"median": float(np.median(per_step)), "min": float(per_step.min()),
                  "p90": float(np.percentile(per_step, 90))}
    for e in evs:
        for v in e:
            hip.hipEventDestroy(v)

    ms_per_step = elapsed * 1e3 / steps
    value = cfg.T * steps / elapsed
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

    # the same layer with an fp32 output (the primary parity bar of bf16
    # layers), for the parity sample below
    out32 = None
    if not args.no_cpu_baseline and cfg.out_dtype != 0 and not args.ring:
        p32 = B.problem_of(cfg, block_m=args.block_m, out_dtype=0, w_layout=layout)
        out32 = B.out_tensor(cfg, out_dtype=0)
        step(None, out32, p32)
        torch.cuda.synchronize()

    dtype = {0: "f32", 1: "bf16", 2: "fp8e4m3", 3: "mxfp4xmxfp8"}[cfg.w_dtype]
    rec = {
        "value": value, "unit": "tokens/s", "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "dtype": dtype,
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f, "E": cfg.E,
                   "top_k": cfg.k, "n_shared": cfg.n_shared, "parallelism": "single GPU",
                   "gemms": "one launch, h ring" if args.ring else "two launches"},
        "roofline": roof, "cpu_baseline": None, "stages_ms": stage_ms, "layer": layer,
        "sustained_clock_mhz": sustained, "parity_sample": None,
        "weight_pack_ms": None if args.stated_weights else pack_s * 1e3,
        "weights": "stated [K][N] layout, no pack" if args.stated_weights else "packed [N][K]",
    }
    del packed, ws
    held = {"inp": inp, "out": out, "out32": out32}

    def finish():
        if not args.no_cpu_baseline:
            _say(f"{cfg.name}: CPU oracle baseline (~{cpu_seconds:.0f} s)")
            rec["cpu_baseline"], rec["parity_sample"] = _cpu_baseline(
                cfg, held["inp"], held["out"], held["out32"], cpu_seconds)
        held.clear()
        _free(torch)
        return rec

    return rec, finish


# the other stated workloads of a default run; their GPU phases run after the
# headline one's (see main)
OTHER_CONFIGS = ["tiny_fp32", "decode_bf16", "skewed_bf16", "prefill_fp8"]


def blas_calibration(reps=50):
    """TFLOP/s of torch.matmul (hipBLASLt) on plain bf16 GEMMs: the prefill
    layer's W1/W3 stage as one dense GEMM (T*k x d times d x 2f), its W2
    stage (T*k x f times f x d) and 8192^3; a reference for what a vendor
    GEMM reaches on the same shapes, without the gather, grouping or
    SwiGLU."""
    import torch

    out = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, (m, k, n) in {"prefill_w13_dense": (32768, 2048, 4096),
                            "prefill_w2_dense": (32768, 2048, 2048),
                            "square_8192": (8192, 8192, 8192)}.items():
        a = torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16)
        b = torch.randn((k, n), generator=g, device="cuda").to(torch.bfloat16)
        for _ in range(10):
            c = torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * m * k * n / (ms * 1e-3) / 1e12
        out[name] = {"m": m, "k": k, "n": n, "ms": ms, "tflops": tf,
                     "frac_of_bf16_peak": tf / 2516.6}
        del a, b, c
    return {"blas_calibration": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 50 warm-up steps: the shader clock ramps up over the first ~50 ms of
    # load (prefill_bf16 GEMMs at ~2.08 GHz after 5 steps, ~2.23 GHz after 50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--other-cpu-seconds", type=float, default=8.0,
                    help="CPU-oracle seconds for each of the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="measure only --workload (by default the other stated workloads "
                         "are measured too, after the headline one, each in a block of "
                         "its own)")
    ap.add_argument("--block-m", type=int, default=0, help="expert tile height (0 = auto)")
    ap.add_argument("--stated-weights", action="store_true",
                    help="pass the weights in the layouts the workloads state ([E][d][f], "
                         "[E][f][d]) instead of packing them once")
    ap.add_argument("--ring", action="store_true",
                    help="time moe_forward_ring (both GEMMs in one launch, h in a bounded ring)")
    ap.add_argument("--blas-calibration", action="store_true",
                    help="time torch.matmul (hipBLASLt) on plain bf16 GEMMs of the prefill "
                         "W1/W3 and W2 shapes and on 8192^3, as a reference for the grouped GEMMs")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="print per-kernel mean counter values of a rocprofv3 --pmc csv (no GPU "
                         "use)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print a per-kernel summary of a rocprofv3 kernel trace of a bench run "
                         "made with the same --steps/--warmup/--workload flags (no GPU use)")
    args = ap.parse_args()
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return
    if args.trace_summary:
        wls = [args.workload]
        if not args.no_other_configs and not args.ring and args.workload == "prefill_bf16":
            wls += OTHER_CONFIGS  # the order main() runs their GPU phases in
        print(trace_summary(args.trace_summary, args.warmup, args.steps, wls))
        return
    if args.blas_calibration:
        print(json.dumps(blas_calibration()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_softmax_amd import binding as B
    from mixture_experts_layer_softmax_amd.configs import CONFIGS

    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    B.load()
    hip = _hip()
    copy_gbps = _copy_gbps(torch)
    # GPU phases first, back to back, the headline workload first; then the
    # CPU-oracle baselines, which launch no kernels.  The shader clock a workload
    # runs at depends on what ran before it (it climbs over the first ~50 ms
    # of a heavy load and sits lower after the FP8 layer's run), so the
    # headline layer runs on a GPU that nothing else has loaded in this
    # process, and every workload gets exactly `warmup` untimed steps of its
    # own before its `steps` timed ones.
    head, head_finish = measure(cfg, args, args.steps, args.warmup, args.cpu_seconds, hip,
                                copy_gbps)
    pending = []
    if not args.no_other_configs and not args.ring and args.workload == "prefill_bf16":
        for name in OTHER_CONFIGS:
            pending.append((name, *measure(CONFIGS[name], args, args.steps, args.warmup,
                                           args.other_cpu_seconds, hip, copy_gbps)))
    head_finish()
    others = {}
    for name, rec, finish in pending:
        finish()
        rec.pop("layer", None)
        others[name] = rec

    device = _device_info()
    device["sustained_clock_mhz"] = head.pop("sustained_clock_mhz")
    device["measured_copy_GBps"] = copy_gbps
    line = {
        "metric": "MoE-layer tokens/s on 1 MI355X; MFMA % peak (prefill), HBM GB/s (decode)",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "stages_ms": head["stages_ms"],
        "layer": head["layer"],
        "device": device,
        "parity_sample": head["parity_sample"],
        "weight_pack_ms": head["weight_pack_ms"],
    }
    if others:
        line["configs"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
