#!/usr/bin/env python3
"""Benchmark of the attention forward hot path on one MI355X.

One step = one ``fa_fwd`` launch over one batch of synthetic input of the
chosen workload (default: 16x8 heads of a 20x20 map, N=400, d=64, bf16).
Inputs are resident in HBM before timing; R rotating input sets (>= 512 MB
in total) keep the 256 MB Infinity Cache from serving them between steps.
The K timed launches are captured once in a HIP graph and replayed, so the
host's launch overhead cannot starve the GPU; HIP events recorded on the
launch stream give the average kernel duration used for the roofline. After
the W warmup steps, untimed replays run for --settle seconds: kernel times
keep falling for tens of milliseconds after a burst starts (clocks, address
translation), and the timed steps should see the steady state.

Prints ONE JSON line on stdout (details go to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_fa2_amd import accounting as acc  # noqa: E402
from exact_attention_fa2_amd import inputs  # noqa: E402

DEFAULT_WORKLOAD = "n400_batched"
METRIC = "attn fwd TFLOP/s (4·B·H·N²·d) and % of MFMA peak / HBM GB/s, N=400..8192"
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the files the forward kernels are built from (code, dispatch, build options)
FWD_SOURCES = ("csrc/fa_device.h", "csrc/fa_fwd_kernel.h", "csrc/fa_fwd.hip", "csrc/fa_fwd_split.h",
               "csrc/fa_fwd_launch.h", "csrc/fa_fwd_small.hip", "build.py")


def kernel_source_hash() -> str:
    """Hash of the forward kernel's sources: stored HBM counters are used only
    while it matches."""
    h = hashlib.sha256()
    for name in FWD_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_fa2_amd", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w: inputs.Workload, budget_s: float):
    """Times the fp64 oracle on the host on a bounded sample of the workload."""
    import numpy as np
    import threadpoolctl

    import oracle

    q, k, v = inputs.make_workload(w, seed=0)
    qd, kd, vd = (oracle.decode(inputs.bits(x), w.dtype) for x in (q, k, v))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    # sample: whole (batch, head) slices taken in order (wrapping around), until
    # the time budget is spent; at least one slice
    done, t0 = 0, time.perf_counter()
    while True:
        b, h = heads[done % len(heads)]
        oracle.attention_fwd(qd[b:b + 1, h:h + 1], kd[b:b + 1, h:h + 1], vd[b:b + 1, h:h + 1], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = acc.metric_flops(1, done, w.N, w.d)
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} (batch, head) slices (the workload has {len(heads)}) of {w.name} "
                  f"(N={w.N}, d={w.d}), fp64 numpy/OpenBLAS, {dt:.1f} s",
    }


def copy_bandwidth(torch, dev, stream, mib: int = 256, reps: int = 20) -> float:
    """GB/s of a plain device-to-device copy (bytes read + bytes written), timed
    with HIP events on `stream`: the bandwidth an HBM-bound kernel can reach
    in practice, reported beside the 8 TB/s peak."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def bench_varlen(args, torch, fa, dev) -> int:
    """Packed variable-length batch through fa_fwd_varlen (same timing scheme)."""
    vm = inputs.VARLEN_MIX
    seqlens, H, d = vm["seqlens"], vm["H"], vm["d"]
    T = sum(seqlens)
    aflops = sum(acc.alg_flops(1, H, n, d, vm["causal"]) for n in seqlens)
    abytes = acc.alg_bytes(1, H, T, d)
    R = max(1, math.ceil(ROTATE_BYTES / abytes))
    sets = []
    for r in range(R):
        q, k, v, cu = inputs.make_varlen(seqlens, H, d, vm["dtype"], seed=r)
        q, k, v, cu = (t.to(dev) for t in (q, k, v, cu))
        sets.append((q, k, v, cu, torch.empty_like(q), torch.empty((H, T), dtype=torch.float32, device=dev)))
    scale = d ** -0.5
    stream = torch.cuda.Stream()

    def launch(i):
        q, k, v, cu, o, lse = sets[i % R]
        fa.fa_fwd_varlen(q, k, v, o, lse, cu, len(seqlens), T, max(seqlens), H, d, scale, vm["causal"])

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            launch(i)
    torch.cuda.synchronize()
    K = args.steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(K):
            launch(i)
    torch.cuda.synchronize()
    t_set = time.perf_counter()
    while time.perf_counter() - t_set < args.settle:
        graph.replay()
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_s = ev0.elapsed_time(ev1) * 1e-3 / K
    log(f"varlen_mix: {len(seqlens)} sequences {sorted(set(seqlens))}, T={T}, H={H}, d={d}: kernel avg "
        f"{kern_s*1e6:.2f} us; {aflops/kern_s/1e12:.1f} TFLOP/s alg")
    print(json.dumps({
        "metric": "attn fwd TFLOP/s, packed variable-length batch", "value": round(aflops / (wall / K) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": vm["dtype"], "data": "synthetic",
        "config": {"workload": "varlen_mix", "seqlens": seqlens, "H": H, "d": d, "input_sets": R},
        "roofline": {"bound": "mfma", "achieved": round(aflops / kern_s / 1e12, 2),
                     "peak": acc.MFMA_PEAK_TFLOPS_16BIT, "unit": "TFLOP/s",
                     "frac": round(aflops / kern_s / 1e12 / acc.MFMA_PEAK_TFLOPS_16BIT, 4), "traffic": None,
                     "kernel": "fa_fwd_varlen", "kernel_us": round(kern_s * 1e6, 3)}}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(inputs.WORKLOADS) + ["varlen_mix"])
    ap.add_argument("--layout", default="bhnd", choices=["bhnd", "bnhd", "qkvpacked"],
                    help="tensor layout at the boundary (fa_fwd / fa_fwd_strided)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--eager", action="store_true", help="launch from Python each step (no graph)")
    ap.add_argument("--warm-cache", action="store_true", help="one input set (cache-resident)")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps after the warmup, so that clocks and address "
                         "translation reach steady state before the timed steps")
    ap.add_argument("--impl", default="fa2", choices=["fa2", "fa1_order", "bwd"],
                    help="fa2: fa_fwd (default); fa1_order: the FlashAttention-1 loop-order "
                         "ablation; bwd: fa_bwd (the backward by recomputation)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="run only a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; the path shards over (batch, head) "
              "with no exchange, so run N=1 (see the sharding design).", file=sys.stderr)
        return 2

    import torch
    import exact_attention_fa2_amd as fa

    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", "0")))
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes x3")
        return 0

    if args.workload == "varlen_mix":
        return bench_varlen(args, torch, fa, dev)
    w = inputs.WORKLOADS[args.workload]
    elem = 2
    abytes = acc.alg_bytes(w.B, w.H, w.N, w.d, elem)
    aflops = acc.alg_flops(w.B, w.H, w.N, w.d, w.causal)
    mflops = acc.metric_flops(w.B, w.H, w.N, w.d)
    metric = METRIC
    if args.impl == "bwd":
        # backward: five N x N x d products (S, dP, dV, dK, dQ) = 2.5x the forward;
        # bytes: read Q, K, V, O, dO and LSE, write dQ, dK, dV
        aflops, mflops = int(2.5 * aflops), int(2.5 * mflops)
        abytes = acc.alg_bytes_bwd(w.B, w.H, w.N, w.d, elem)
        metric = "attn bwd TFLOP/s (2.5 x 4·B·H·N²·d)"
    R = 1 if args.warm_cache else max(1, math.ceil(ROTATE_BYTES / abytes))
    log(f"workload {w.name}: {w.describe()}; {R} rotating input sets; alg bytes {abytes/1e6:.2f} MB, "
        f"alg flop {aflops/1e9:.2f} G")

    sets = []
    for r in range(R):
        q, k, v = (t.to(dev) for t in inputs.make_workload(w, seed=r))
        if args.layout == "bnhd":
            q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        elif args.layout == "qkvpacked":
            qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()
            q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        o = torch.empty_like(q) if args.layout == "bhnd" else torch.empty(
            (w.B, w.N, w.H, w.d), dtype=q.dtype, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        sets.append((q, k, v, o, lse))
    stream = torch.cuda.Stream()
    ws = None
    grads = []
    if args.impl == "fa1_order":
        ws = torch.empty(fa.fa_fwd_fa1_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    elif args.impl == "bwd":
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
        for r, (q, k, v, o, lse) in enumerate(sets):
            fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal)  # O, LSE (untimed)
            do = inputs.make_like(q.cpu(), 1000 + r).to(dev)
            grads.append((do, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)))
        torch.cuda.synchronize()

    def launch(i):
        q, k, v, o, lse = sets[i % R]
        if args.impl == "fa2" and args.layout != "bhnd":
            st = fa._strides_bnhd
            fa.fa_fwd_strided(q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal,
                              st(q), st(k), st(v), st(o))
        elif args.impl == "fa2":
            fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal)
        elif args.impl == "fa1_order":
            fa.fa_fwd_fa1_order(q, k, v, o, lse, ws, w.B, w.H, w.N, w.d, w.scale, w.causal)
        else:
            do, dq, dk, dv = grads[i % R]
            fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, w.B, w.H, w.N, w.d, w.scale, w.causal)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            launch(i)
    torch.cuda.synchronize()
    out_idx = sets[0][3] if args.impl != "bwd" else grads[0][1]
    ref_o = out_idx.clone()

    K = args.steps
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(K):
                launch(i)
        torch.cuda.synchronize()
        graph.replay()  # untimed replay: check the graph reproduces the eager output
        torch.cuda.synchronize()
        if not torch.equal(out_idx, ref_o):
            log("graph replay disagrees with the eager launch")
            return 1

    # untimed settle phase: the same steps until `settle` seconds have passed
    t_set = time.perf_counter()
    with torch.cuda.stream(stream):
        while time.perf_counter() - t_set < args.settle:
            if graph is not None:
                graph.replay()
            else:
                for i in range(K):
                    launch(i)
            torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                launch(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)

    ms_per_step = wall * 1e3 / K
    kern_s = ev_ms * 1e-3 / K  # average launch duration on the launch stream
    value = mflops / (ms_per_step * 1e-3) / 1e12
    intensity = aflops / abytes
    ridge = acc.MFMA_PEAK_TFLOPS_16BIT * 1e12 / (acc.HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        achieved, peak, unit, bound = abytes / kern_s / 1e9, acc.HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = aflops / kern_s / 1e12, acc.MFMA_PEAK_TFLOPS_16BIT, "TFLOP/s", "mfma"
    log(f"ms/step {ms_per_step:.4f} (wall), kernel avg {kern_s*1e6:.2f} us (events); "
        f"{aflops/kern_s/1e12:.1f} TFLOP/s alg, {abytes/kern_s/1e9:.0f} GB/s alg")

    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "input_sets": R, "graph": graph is not None, "impl": args.impl, "layout": args.layout,
                   "settle_s": args.settle,
                   "parallelism": "none (1 GPU)"},
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": stored_traffic(w.name) if args.impl == "fa2" else None,
            "kernel": {"fa2": "fa_fwd", "fa1_order": "fa_fwd_fa1_kernel",
                       "bwd": "fa_bwd (dot + dK/dV + dQ kernels)"}[args.impl],
            "kernel_us": round(kern_s * 1e6, 3),
            "alg_bytes": abytes,
            "alg_flop": aflops,
        },
    }
    if w.causal:
        out["roofline"]["note"] = ("value uses the metric's 4·B·H·N²·d, which counts the masked "
                                   "half of a causal problem; achieved counts only the computed half")
    if bound == "hbm":
        # the rate a plain copy reaches on this GPU, timed in the same run
        cgbs = copy_bandwidth(torch, dev, stream)
        out["roofline"]["copy_gbs"] = round(cgbs, 1)
        out["roofline"]["frac_of_copy"] = round(achieved / cgbs, 4)
        log(f"device copy {cgbs:.0f} GB/s; kernel reaches {achieved / cgbs:.1%} of it")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
