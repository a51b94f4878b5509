#!/usr/bin/env python3
"""Throughput of the FAVOR+ forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload text_bidir]

A step is one forward call (favor_fwd_bidir or favor_fwd_causal) over one
batch of synthetic inputs of the workload's shape, inputs already resident in
HBM.  Calls rotate over several input/output buffer sets (>= 1 GiB in total,
four times the 256 MiB last-level cache) so that the timing is an HBM
measurement, not a cache one.  W steps are run untimed, then exactly K steps
are timed between two events recorded on the stream the kernels run on, with
a device synchronisation on both sides.

Prints one JSON line (rank 0 = the only rank).  Metric: tokens*heads/s of the
forward pass at B8 H8 L4096 d64 m256 (the text-length bidirectional workload),
with the roofline of the path and the fp64 CPU oracle timed on a bounded
sample of the same workload beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="text_bidir")
    ap.add_argument("--causal", action="store_true", help="time the causal form of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU oracle sample")
    ap.add_argument("--cache-hot", action="store_true",
                    help="reuse one buffer set (a cache measurement, labelled as such)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_kernelized_attention_favor_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".cpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, causal: bool):
    """HBM bytes per call from the committed rocprofv3 counter summary, or None.

    None when no summary exists for this workload or when the kernel sources
    changed since the counters were taken.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{workload}{'-causal' if causal else ''}"
    e = t.get(key)
    if not e or e.get("kernel_src_digest") != kernel_source_digest():
        return None
    return e.get("bytes_per_call")


def cpu_baseline(w, seconds: float):
    """Time the fp64 oracle on whole heads of the same workload (host cores)."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    W = oracle.draw_w(w.seed_w, w.m, w.d)
    f = oracle.causal if w.causal else oracle.bidir
    heads = 0
    spent = 0.0
    # One head's inputs from the host generator (drawn outside the timing);
    # the oracle's cost does not depend on the values, so every timed head
    # reuses them.
    q, k, v = (t.double().numpy()[0, 0] for t in workloads.host_qkv(w, heads=[0]))
    while spent < seconds and heads < w.heads:
        t0 = time.perf_counter()
        f(q, k, v, W)
        spent += time.perf_counter() - t0
        heads += 1
    tok = heads * w.L
    return {"value": tok / spent, "unit": "tokens*heads/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {w.heads} heads of {w.name} (L={w.L}, d={w.d}, m={w.m}, "
                      f"{'causal' if w.causal else 'bidirectional'}), fp64 numpy, "
                      f"{spent:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the forward pass is not sharded across GPUs in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_kernelized_attention_favor_amd as fv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = workloads.workload(args.workload)
    if args.causal:
        w = w.with_(causal=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # Projection: the library's host draw, uploaded once.
    W = torch.from_numpy(fv.draw_projection(w.seed_w, w.m, w.d)).to(dev)

    elem = 2 if w.dtype == "bf16" else 4
    set_bytes = 4 * w.heads * w.L * w.d * elem
    nsets = 1 if args.cache_hot else max(1, -(-(1 << 30) // set_bytes))
    sets = []
    for i in range(nsets):
        q, k, v = workloads.device_qkv(w, seed=w.seed_in + 7919 * i)
        sets.append((q, k, v, torch.empty_like(q)))
    ws = torch.empty(fv.workspace_bytes(w.B, w.H, w.L, w.d, w.m, fv.BF16 if w.dtype == "bf16"
                                        else fv.F32, w.causal), dtype=torch.uint8, device=dev)
    fwd = fv.fwd_causal if w.causal else fv.fwd_bidir
    stream = torch.cuda.current_stream(dev)

    def step(i):
        q, k, v, o = sets[i % nsets]
        fwd(q, k, v, W, out=o, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps

    tokens = w.heads * w.L
    value = tokens / (ms * 1e-3)
    alg_bytes = 4 * w.heads * w.L * w.d * elem                 # Q, K, V read + O written once
    alg_flops = 8.0 * w.heads * w.L * w.d * w.m
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    achieved_tflops = alg_flops / (ms * 1e-3) / 1e12
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg_flops / (BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / BF16_PEAK_TFLOPS, 4)}
    tr = measured_traffic(w.name, w.causal)
    roof["traffic"] = tr
    roof["scope"] = "whole forward call (all kernels of one step)"

    out = {
        "metric": "FAVOR+ fwd tokens*heads/s + % of roofline, B8 H8 L4096 d64 m256",
        "value": round(value, 1),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q, K, V; orthogonal Gaussian W)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "m": w.m,
                   "causal": w.causal, "buffer_sets": nsets,
                   "cache": "hot" if args.cache_hot else "rotating >= 1 GiB"},
        "tflops_alg": round(achieved_tflops, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
