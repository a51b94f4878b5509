#!/usr/bin/env python3
"""Throughput of the FAVOR+ forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload text_bidir] [--pass bwd]

A step is one forward call (favor_fwd_bidir or favor_fwd_causal) over one
batch of synthetic inputs of the workload's shape, inputs already resident in
HBM; with --pass bwd, one backward call (favor_bwd_attn: dQ, dK, dV for a
seeded upstream gradient dO, the forward's state recomputed inside); with
--pass prefill, one causal favor_prefill call exporting the state (--carry:
continuing a carried state); with
--pass decode, one favor_decode call (one new token for each of the B*H heads,
the state updated in place).  Calls rotate over several input/output buffer sets (>= 1 GiB in total,
four times the 256 MiB last-level cache) so that the timing is an HBM
measurement, not a cache one.  W steps are run untimed, then exactly K steps
are timed between two events recorded on the stream the kernels run on, with
a device synchronisation on both sides.

Prints one JSON line (rank 0 = the only rank).  Metric: tokens*heads/s of the
forward pass at B8 H8 L4096 d64 m256 (the text-length bidirectional workload),
with the roofline of the dominant kernel (its algorithmic bytes or flops per
launch over its average duration from HIP events, in a second pass of the
same K steps), the whole call's roofline, and the fp64 CPU oracle timed on a
bounded sample of the same workload beside it.

Measurement helpers: --copy-calibration runs a plain device copy of known size
(the reference for the HBM byte counters); --pmc-summary DIR turns rocprofv3
FETCH_SIZE / WRITE_SIZE passes into profiles/traffic.json.
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
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector FMA, published (256 CUs at 2.4 GHz)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (a few hundred untimed calls first: the clocks settle within ~10 ms of
    # continuous work; 500 timed calls of the text workload take ~35 ms)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="text_bidir")
    ap.add_argument("--causal", action="store_true", help="time the causal form of the workload")
    ap.add_argument("--kernel", choices=("softmax", "gaussian", "relu"), default="softmax",
                    help="attention kernel the features estimate (default softmax)")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd", "prefill", "decode"),
                    default="fwd",
                    help="time the forward (default), the backward pass, the causal prefill "
                         "that exports its state, or one decoding step per head")
    ap.add_argument("--carry", action="store_true",
                    help="with --pass prefill: continue a carried state (the state a prefill "
                         "of the same shape exported) instead of starting empty")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU oracle sample")
    ap.add_argument("--cache-hot", action="store_true",
                    help="reuse one buffer set (a cache measurement, labelled as such)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain fp32 device copy of known size (the reference "
                         "kernel that scales the HBM byte counters)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE passes found under "
                         "DIR/{fetch,write,copy_fetch,copy_write} into profiles/traffic.json")
    return ap.parse_args()


# The sources the forward pass's counted kernels are compiled from: a change
# to any of them voids the committed counter summary.
FORWARD_SOURCES = ("kernels_mfma.hip", "kernels_fused.hip", "mfma_common.h", "favor_internal.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_kernelized_attention_favor_amd", "csrc")
    for f in sorted(FORWARD_SOURCES):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_counters(workload: str, causal: bool, kernel: str):
    """Executed-MFMA fraction of the bf16 peak of `kernel` from the committed
    counter summary (its own rocprofv3 duration), or None (absent or stale)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(f"{workload}{'-causal' if causal else ''}")
    if not e or e.get("kernel_src_digest") != kernel_source_digest():
        return None
    return e.get("kernels", {}).get(kernel, {}).get("mfma_frac")


def measured_traffic(workload: str, causal: bool, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None.

    None when no summary exists for this workload and kernel, or when the
    kernel sources changed since the counters were taken.
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
    k = e.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def kernel_work(name: str, w, nseg: int, seg: int, elem: int, backward: bool = False):
    """Algorithmic (bytes, flops) of one launch of a kernel of the path.

    The whole path moves 4 d elements per token*head (Q, K, V read, O
    written once: 8 d bytes in bf16) and does 8 d m flops (two projections
    and two m x (d+1) contractions).  A key-side kernel owns the K and V
    reads and the key projection and contraction (2 d elements, 4 d m flops
    per token*head it covers), a query-side kernel the Q read, O write,
    query projection and contraction (the same), the causal scan both.
    Combine and prefix kernels only touch workspace: no algorithmic bytes or
    flops.
    """
    th = w.heads * w.L
    # Backward (favor_bwd_attn): Q, K, V, dO read and dQ, dK, dV written once
    # (7 d elements per token*head); 22 d m flops: the key state (4 d m),
    # the query side (projection, [num | den], T, dq: 8 d m), the query
    # state from the features (2 d m) and the key side (projection, H, dk,
    # dv: 8 d m).
    bwd = {"gb_query": (3, 8.0), "gb_gstate": (0, 2.0), "gb_key": (2, 8.0),
           # matrix-core backward: bquery forms the features, [num | den], T, dq
           # and the query state G (10 d m); bkey the key features, H, dk, dv
           "bquery": (3, 10.0), "bkey": (2, 8.0),
           # the same work split into passes that each rebuild the features:
           # 1/den and u0 (projection, [num | den]), dq (projection, T, dq),
           # the query state (projection, G); dk (projection, H, dk), dv
           # (projection, dv)
           "bq_den": (2, 4.0), "bq_dq": (1, 6.0), "bq_g": (0, 4.0),
           "bkey_dk": (1, 6.0), "bkey_dv": (1, 4.0),
           # causal matrix-core backward (kpart or ckey owns the K, V reads and the
           # key state): the scan for (L, p) reads Q and dO (both
           # projections, [num | den], the state update: 8 d m); dq (both
           # projections, T, state update, dq: 10 d m); the segments' query
           # states (projection, G: 4 d m); dk (both projections, H, G
           # update, dk: 10 d m); dv (key projection, the query projection
           # twice, dv, G update: 10 d m); masked in-chunk terms uncounted
           "cscan_lp": (2, 8.0), "cbq": (1, 10.0), "cbg": (0, 4.0),
           "cbk_dk": (1, 10.0), "cbk_dv": (1, 10.0)}
    if name == "g_decode":
        # one token per head: the state [m][d+4] fp32 read and written, q, k,
        # v read and o written; two projections, the state update and the
        # contraction (8 d m flops)
        return (w.heads * (2 * w.m * (w.d + 4) * 4 + 4 * w.d * elem), 8.0 * w.d * w.m * w.heads)
    if name in bwd:
        nb, nf = bwd[name]
        return (nb * w.d * elem * th, nf * w.d * w.m * th)
    half = (2 * w.d * elem * th, 4.0 * w.d * w.m * th)
    if backward:
        # the backward's key state: kpart, ckey or g_state reads K and V once
        return half if name in ("kpart", "ckey", "g_state") else (0, 0.0)
    if w.causal:
        # The causal scan reads Q, K, V and writes O and does both projections
        # and both contractions: the whole path's algorithmic work.  The
        # segment-state pass before it (ckey, kpart, g_state) re-reads K and V and
        # recomputes the key side: overhead, credited nothing, so that the
        # kernels' bytes sum to 4 d elements per token*head.
        if name in ("cscan", "g_apply"):
            return (2 * half[0], 2 * half[1])
        return (0, 0.0)
    if name in ("kpart", "qapply", "qstream", "g_state", "g_apply"):
        return half
    if name == "fused":
        # the persistent bidirectional kernel: both sides, the whole path's
        # algorithmic work (fprep, before it, only converts W)
        return (2 * half[0], 2 * half[1])
    return (0, 0.0)


def cpu_baseline(w, seconds: float, kernel: str = "softmax", backward: bool = False):
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
    if backward:
        fb = oracle.causal_backward if w.causal else oracle.bidir_backward
        rng = np.random.default_rng(w.seed_in + 5)
        dO = rng.standard_normal((w.L, w.d))
        f = lambda q, k, v, W, kernel: fb(q, k, v, W, dO, kernel)
    heads = 0
    spent = 0.0
    # One head's inputs from the host generator (drawn outside the timing);
    # the oracle's cost does not depend on the values, so every timed head
    # reuses them.
    q, k, v = (t.double().numpy()[0, 0] for t in workloads.host_qkv(w, heads=[0]))
    # Heads in workload order, passes over the workload repeated until the
    # time budget is spent (a pass shorter than the budget is timed several
    # times over), the last pass possibly partial.
    while spent < seconds:
        t0 = time.perf_counter()
        f(q, k, v, W, kernel=kernel)
        spent += time.perf_counter() - t0
        heads += 1
    tok = heads * w.L
    passes = heads / w.heads
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": tok / spent, "unit": "tokens*heads/s", "cores": int(threads),
            "host_cores": len(os.sched_getaffinity(0)), "cpu_model": model,
            "kind": "oracle",
            "sample": f"{heads} head evaluations ({passes:.2f} passes over the {w.heads} heads) "
                      f"of {w.name} ({'backward, ' if backward else ''}"
                      f"{kernel} kernel, L={w.L}, d={w.d}, m={w.m}, "
                      f"{'causal' if w.causal else 'bidirectional'}), fp64 numpy, "
                      f"{spent:.1f} s"}


COPY_ELEMS = 1 << 28          # fp32 elements of the calibration copy (1 GiB read, 1 GiB written)


def copy_ceiling(reps: int = 20):
    """Measured HBM ceiling: a plain device copy (dst = -src, fp32, 1 GiB read and
    1 GiB written) timed with events over `reps` back-to-back launches, outside
    any profiler.  Returns {"GB_s", "ms", "bytes", "kernel"}."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 8 * COPY_ELEMS
    del src, dst
    torch.cuda.empty_cache()
    return {"GB_s": round(nbytes / ms / 1e6, 1), "ms": round(ms, 4), "bytes": nbytes,
            "kernel": "torch.neg fp32, 1 GiB read + 1 GiB written, 20 launches"}


def copy_calibration(steps: int):
    """A plain device copy (dst = -src, fp32) of COPY_ELEMS elements, `steps` times."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_calibration": True, "bytes_read": 4 * COPY_ELEMS,
                      "bytes_written": 4 * COPY_ELEMS, "ms": round(ms, 4),
                      "GB_s": round(8 * COPY_ELEMS / ms / 1e6, 1)}), flush=True)


FAVOR_KERNELS = ("fprep", "fused", "ckey", "kpart", "kcombine", "qapply", "qstream", "kprefix", "cscan", "g_state",
                 "g_combine", "g_apply", "gb_query", "gb_gstate", "gb_gcombine", "gb_key",
                 "bprep", "bcombine", "bqr", "gcombine", "bkeyr", "sexport", "g_decode",
                 "g_state_reset", "draw_block", "g_feature_map", "cbq", "cbg", "cbsuffix")
# passes of the templated backward kernels, by their third template argument
_PASSES = {"bqr": ("bq_den", "bq_dq", "bq_g"), "bkeyr": ("bkey_dk", "bkey_dv"),
           "cbk": ("cbk_dk", "cbk_dv")}


def _favor_kernel(name: str):
    """Short name of a libfavor kernel from a demangled or mangled symbol, else None."""
    import re
    m = re.search(r"favor::\(anonymous namespace\)::(\w+)(?:<([^>]*)>)?\(", name)
    if m:
        k, targs = m.group(1), m.group(2) or ""
        args = [a.strip() for a in targs.split(",")] if targs else []
    else:   # _ZN5favor12_GLOBAL__N_1<len><name>I<L..E>...E
        m = re.search(r"_ZN5favor12_GLOBAL__N_1(\d+)", name)
        k = name[m.end():m.end() + int(m.group(1))] if m else None
        rest = name[m.end() + int(m.group(1)):] if m else ""
        args = re.findall(r"L[a-z](\d+)E", rest.split("EEv")[0] + "E") if rest.startswith("I") else []
    if k in _PASSES and len(args) >= 3 and args[2].isdigit():
        return _PASSES[k][int(args[2])]
    if k == "cscan":   # the backward's variant (last template argument true)
        tail = (m.group(2) or "") if "(anonymous namespace)" in name else name[m.end():]
        if re.search(r"true\s*$", tail) or re.search(r"ELb1EE", tail):
            return "cscan_lp"
    return k if k in FAVOR_KERNELS else None


def _pmc_rows(d):
    """(kernel short name, counter, value) per dispatch from a rocprofv3 CSV tree."""
    import csv
    import glob
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                n = r["Kernel_Name"]
                k = _favor_kernel(n)
                if k:
                    pass
                elif "neg_kernel" in n or ("neg" in n and "elementwise" in n):
                    k = "copy"
                else:
                    continue
                out.append((k, r["Counter_Name"], float(r["Counter_Value"])))
    return out


def _kernel_avg_ns(stats_dir):
    """Average duration (ns) of each libfavor kernel from a rocprofv3 --stats tree."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = _favor_kernel(r["Name"])
                if k:
                    out[k] = float(r["AverageNs"])
    return out


def _mean_by_kernel(rows, counter):
    acc = {}
    for k, c, v in rows:
        if c == counter:
            acc.setdefault(k, []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def pmc_summary(root: str, workload: str, causal: bool):
    """Per-launch HBM bytes of each kernel, counters scaled by the copy kernel.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) come from separate passes;
    each is multiplied by (known bytes of the calibration copy) / (what the
    same counter reads for it), so the figures are in bytes as the copy
    defines them.
    """
    fetch = _mean_by_kernel(_pmc_rows(os.path.join(root, "fetch")), "FETCH_SIZE")
    write = _mean_by_kernel(_pmc_rows(os.path.join(root, "write")), "WRITE_SIZE")
    cf = _mean_by_kernel(_pmc_rows(os.path.join(root, "copy_fetch")), "FETCH_SIZE")["copy"][0]
    cw = _mean_by_kernel(_pmc_rows(os.path.join(root, "copy_write")), "WRITE_SIZE")["copy"][0]
    f_scale = 4 * COPY_ELEMS / cf
    w_scale = 4 * COPY_ELEMS / cw
    kernels = {}
    lines = [f"copy calibration: {4 * COPY_ELEMS} B read -> FETCH_SIZE {cf:.1f} "
             f"(x{f_scale:.2f}), {4 * COPY_ELEMS} B written -> WRITE_SIZE {cw:.1f} "
             f"(x{w_scale:.2f})",
             f"{'kernel':10s} {'dispatches':>10s} {'FETCH_SIZE':>14s} {'WRITE_SIZE':>14s} "
             f"{'fetch MB':>10s} {'write MB':>10s} {'total MB':>10s}"]
    for k in FAVOR_KERNELS:
        if k not in fetch or k not in write:
            continue
        fb = fetch[k][0] * f_scale
        wb = write[k][0] * w_scale
        kernels[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                      "bytes_per_launch": round(fb + wb), "dispatches": fetch[k][1]}
        lines.append(f"{k:10s} {fetch[k][1]:10d} {fetch[k][0]:14.1f} {write[k][0]:14.1f} "
                     f"{fb / 1e6:10.2f} {wb / 1e6:10.2f} {(fb + wb) / 1e6:10.2f}")
    # Matrix-core and transcendental work from a third pass (when present):
    # SQ_INSTS_VALU_MFMA_MOPS_* count 512-flop units of executed MFMA work,
    # SQ_INSTS_VALU_TRANS_F32 wave-level transcendental instructions (the
    # exponentials); rates use each kernel's average duration from the
    # kernel-trace pass in the same directory.
    mfma_dir = os.path.join(root, "mfma")
    if os.path.isdir(mfma_dir):
        rows = _pmc_rows(mfma_dir)
        bf = _mean_by_kernel(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        hf = _mean_by_kernel(rows, "SQ_INSTS_VALU_MFMA_MOPS_F16")
        tr = _mean_by_kernel(rows, "SQ_INSTS_VALU_TRANS_F32")
        dur = _kernel_avg_ns(os.path.join(root, "stats"))
        lines.append(f"{'kernel':10s} {'MFMA GFLOP':>11s} {'avg us':>8s} {'TFLOP/s':>9s} "
                     f"{'of 2.5 PF':>9s} {'exp insts':>10s}")
        for k, e in kernels.items():
            if k not in bf:
                continue
            fl = 512.0 * (bf[k][0] + hf.get(k, (0.0, 0))[0])
            e["mfma_flops_executed"] = round(fl)
            e["trans_insts"] = round(tr.get(k, (0.0, 0))[0])
            if k in dur:
                tf = fl / dur[k] / 1e3
                e["avg_us"] = round(dur[k] / 1e3, 3)
                e["mfma_tflops_executed"] = round(tf, 1)
                e["mfma_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
                lines.append(f"{k:10s} {fl / 1e9:11.2f} {dur[k] / 1e3:8.2f} {tf:9.1f} "
                             f"{tf / BF16_PEAK_TFLOPS:9.3f} {e['trans_insts']:10d}")
    key = f"{workload}{'-causal' if causal else ''}"
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        t = {}
    t[key] = {"kernel_src_digest": kernel_source_digest(), "kernels": kernels,
              "fetch_scale": f_scale, "write_scale": w_scale}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("\n".join(lines), flush=True)


def decode_bench(args, w, fv, W, dev, elem):
    """--pass decode: K favor_decode calls (one token per head each) on a
    state filled by the warmup calls; one JSON line like the forward's."""
    import torch
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev).manual_seed(w.seed_in)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    n = 64                                   # token slots cycled through
    toks = [tuple((torch.randn((w.B, w.H, w.d), generator=g, device=dev) * s).to(td)
                  for s in (w.d ** -0.25, w.d ** -0.25, 1.0)) for _ in range(n)]
    outs = [torch.empty((w.B, w.H, w.d), dtype=td, device=dev) for _ in range(n)]
    st = fv.state_new(w.B, w.H, w.d, w.m)

    def step(i):
        q, k, v = toks[i % n]
        fv.decode(q, k, v, W, st, kernel=args.kernel, out=outs[i % n], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps
    # The serving loop's form: n steps captured once in a HIP graph and
    # replayed (no host work per step), the same state advancing.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            q, k, v = toks[i]
            fv.decode(q, k, v, W, st, kernel=args.kernel, out=outs[i])
    reps = max(1, args.steps // n)
    for _ in range(max(1, args.warmup // n)):
        graph.replay()
    torch.cuda.synchronize()
    gs = torch.cuda.current_stream(dev)
    e0.record(gs)
    for _ in range(reps):
        graph.replay()
    e1.record(gs)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n)
    fv.timing_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kt = fv.timing_stop()
    kname = "g_decode"
    tot, launches = kt[kname]
    sec = tot / launches * 1e-3
    nb, nf = kernel_work(kname, w, 1, w.L, elem)
    a = nb / sec / 1e9
    out = {
        "metric": "FAVOR+ causal decode tokens*heads/s, B8 H8 d64 m256",
        "value": round(w.heads / (ms * 1e-3), 1), "unit": "tokens*heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "step_form": f"graph replay ({n} steps per graph, {reps} replays)",
        "eager_ms_per_step": round(ms_eager, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian q, k, v per step; orthogonal Gaussian W)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "m": w.m,
                   "attn_kernel": args.kernel, "pass": "decode"},
        "roofline": {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kname,
                     "kernel_avg_us": round(sec * 1e6, 3)},
        "kernels": {kname: {"avg_us": round(sec * 1e6, 3), "launches": launches,
                                 "alg_bytes": nb, "alg_flops": nf}},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.workload, args.causal)
        return
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
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
    if args.pass_ in ("prefill", "decode"):
        w = w.with_(causal=True)
    if args.pass_ == "decode":
        decode_bench(args, w, fv, W, dev, elem)
        return
    backward = args.pass_ == "bwd"
    set_bytes = (8 if backward else 4) * w.heads * w.L * w.d * elem
    nsets = 1 if args.cache_hot else max(1, -(-(1 << 30) // set_bytes))
    sets = []
    for i in range(nsets):
        q, k, v = workloads.device_qkv(w, seed=w.seed_in + 7919 * i)
        if backward:
            g = torch.Generator(device=dev).manual_seed(w.seed_in + 5 + i)
            do = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
            sets.append((q, k, v, do, tuple(torch.empty_like(q) for _ in range(3))))
        else:
            sets.append((q, k, v, torch.empty_like(q)))
    dt_code = fv.BF16 if w.dtype == "bf16" else fv.F32
    ws_bytes = (fv.bwd_workspace_bytes if backward else fv.workspace_bytes)(
        w.B, w.H, w.L, w.d, w.m, dt_code, w.causal)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fwd_ = fv.fwd_causal if w.causal else fv.fwd_bidir
    stream = torch.cuda.current_stream(dev)
    if args.pass_ == "prefill":
        ws_bytes = fv._binding.prefill_workspace_bytes(w.B, w.H, w.L, w.d, w.m, dt_code)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        st_out = fv.state_new(w.B, w.H, w.d, w.m)
        st_in = None
        if args.carry:
            q0, k0, v0, o0 = sets[0]
            st_in = fv.state_new(w.B, w.H, w.d, w.m)
            fv.prefill(q0, k0, v0, W, state_out=st_in, kernel=args.kernel, out=o0,
                       workspace=ws, stream=stream)

        def fwd(q, k, v, W, out, workspace, stream):
            return fv.prefill(q, k, v, W, state_in=st_in, state_out=st_out, kernel=args.kernel,
                              out=out, workspace=workspace, stream=stream)
    elif backward:
        def fwd(q, k, v, W, out, workspace, stream):
            return fv.bwd(q, k, v, W, out[0], causal=w.causal, kernel=args.kernel, out=out[1],
                          workspace=workspace, stream=stream)
        sets = [(q, k, v, (do, outs)) for (q, k, v, do, outs) in sets]
    else:
        fwd = lambda *a, **kw: fwd_(*a, kernel=args.kernel, **kw)

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

    def timed(calls, pick):
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(calls):
            pick(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls

    # Spread: the same K calls timed five more times (min, median, max), and
    # the cache-hot figure (one buffer set, the inputs resident in the
    # 256 MB last-level cache where they fit), labelled as such.
    reps = sorted(timed(args.steps, step) for _ in range(5))
    q0, k0, v0, o0 = sets[0]
    hot = timed(args.steps, lambda i: fwd(q0, k0, v0, W, out=o0, workspace=ws, stream=stream))
    # Per-kernel durations: the same K steps again, with the library
    # recording a HIP event on `stream` before and after each of its kernel
    # launches.  A second pass, because event records between kernels add a
    # few microseconds of idle time per step that the whole-step figure above
    # must not include.
    torch.cuda.synchronize()
    fv.timing_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kt = fv.timing_stop()

    # Projection redraw (workloads that redraw W every k calls): the same K
    # steps again with a fresh host draw (favor_draw_projection, seed
    # s_W + call // k) uploaded synchronously before every k-th call.
    redraw = None
    if w.redraw_every:
        Wn = torch.empty_like(W)
        t_draw = 0.0
        torch.cuda.synchronize()
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for i in range(args.steps):
            if i % w.redraw_every == 0:
                td = time.perf_counter()
                Wh = torch.from_numpy(fv.draw_projection(w.seed_w + i // w.redraw_every, w.m, w.d))
                t_draw += time.perf_counter() - td
                Wn.copy_(Wh)           # host -> device, ordered on the stream
            q, k, v, o = sets[i % nsets]
            fwd(q, k, v, Wn, out=o, workspace=ws, stream=stream)
        r1.record(stream)
        torch.cuda.synchronize()
        ms_r = r0.elapsed_time(r1) / args.steps
        ndraw = -(-args.steps // w.redraw_every)
        # Overlapped: a host thread draws the next window's W while the
        # current window's calls run; each draw lands in pinned host memory
        # and goes up with a non-blocking copy into the other of two device
        # W buffers, ordered on the stream before the window's first call.
        import concurrent.futures as cf
        Wd = [torch.empty_like(W), torch.empty_like(W)]
        Wp = [torch.empty(W.shape, dtype=W.dtype, pin_memory=True) for _ in range(2)]
        upl = [torch.cuda.Event(), torch.cuda.Event()]
        seed_of = lambda win: w.seed_w + win
        draw = lambda win: fv.draw_projection(seed_of(win), w.m, w.d)
        o0_ = torch.cuda.Event(enable_timing=True)
        o1_ = torch.cuda.Event(enable_timing=True)
        with cf.ThreadPoolExecutor(max_workers=1) as pool:
            # window 0's W is in place before the timed region, window 1's
            # draw already running
            Wp[0].copy_(torch.from_numpy(draw(0)))
            Wd[0].copy_(Wp[0])
            nxt = pool.submit(draw, 1)
            torch.cuda.synchronize()
            o0_.record(stream)
            for i in range(args.steps):
                win = i // w.redraw_every
                if i % w.redraw_every == 0 and win > 0:
                    slot = win % 2
                    upl[slot].synchronize()          # the pinned buffer's last upload is done
                    Wp[slot].copy_(torch.from_numpy(nxt.result()))
                    Wd[slot].copy_(Wp[slot], non_blocking=True)
                    upl[slot].record(stream)
                    nxt = pool.submit(draw, win + 1)
                q, k, v, o = sets[i % nsets]
                fwd(q, k, v, Wd[win % 2], out=o, workspace=ws, stream=stream)
            o1_.record(stream)
            torch.cuda.synchronize()
            nxt.result()
        ms_o = o0_.elapsed_time(o1_) / args.steps
        # On the device: favor_draw_projection_device enqueued on the stream
        # before every k-th call (no host work, no copy).
        torch.cuda.synchronize()
        d0_ = torch.cuda.Event(enable_timing=True)
        d1_ = torch.cuda.Event(enable_timing=True)
        d0_.record(stream)
        for i in range(args.steps):
            if i % w.redraw_every == 0:
                fv.draw_projection_device(w.seed_w + i // w.redraw_every, w.m, w.d, out=Wn,
                                          stream=stream)
            q, k, v, o = sets[i % nsets]
            fwd(q, k, v, Wn, out=o, workspace=ws, stream=stream)
        d1_.record(stream)
        torch.cuda.synchronize()
        ms_d = d0_.elapsed_time(d1_) / args.steps
        # On the device, overlapped: the next window's W drawn on a second
        # stream (default priority) into the other of two buffers while the
        # current window's calls run; the main stream waits for that draw
        # only at the window switch.
        side = torch.cuda.Stream(dev)
        ready = [torch.cuda.Event(), torch.cuda.Event()]
        used = [torch.cuda.Event(), torch.cuda.Event()]
        fv.draw_projection_device(seed_of(0), w.m, w.d, out=Wd[0], stream=stream)
        torch.cuda.synchronize()
        d0_.record(stream)
        for i in range(args.steps):
            win = i // w.redraw_every
            if i % w.redraw_every == 0:
                if win > 0:
                    stream.wait_event(ready[win % 2])
                nxt_slot = (win + 1) % 2
                if win > 0:
                    used[nxt_slot].record(stream)      # the last call that read that buffer
                side.wait_event(used[nxt_slot])
                fv.draw_projection_device(seed_of(win + 1), w.m, w.d, out=Wd[nxt_slot],
                                          stream=side)
                ready[nxt_slot].record(side)
            q, k, v, o = sets[i % nsets]
            fwd(q, k, v, Wd[win % 2], out=o, workspace=ws, stream=stream)
        d1_.record(stream)
        torch.cuda.synchronize()
        ms_do = d0_.elapsed_time(d1_) / args.steps
        ndd = 50
        d0_.record(stream)
        for i in range(ndd):
            fv.draw_projection_device(w.seed_w + i, w.m, w.d, out=Wn, stream=stream)
        d1_.record(stream)
        torch.cuda.synchronize()
        draw_dev_ms = d0_.elapsed_time(d1_) / ndd
        redraw = {"every": w.redraw_every, "ms_per_step": round(ms_r, 5),
                  "overhead_ms_per_step": round(ms_r - ms, 5),
                  "host_draw_ms": round(1e3 * t_draw / ndraw, 3),
                  "overlapped_ms_per_step": round(ms_o, 5),
                  "overlapped_overhead_ms_per_step": round(ms_o - ms, 5),
                  "device_draw_ms": round(draw_dev_ms, 4),
                  "device_ms_per_step": round(ms_d, 5),
                  "device_overhead_ms_per_step": round(ms_d - ms, 5),
                  "device_overlapped_ms_per_step": round(ms_do, 5),
                  "device_overlapped_overhead_ms_per_step": round(ms_do - ms, 5)}

    tokens = w.heads * w.L
    value = tokens / (ms * 1e-3)
    alg_bytes = (7 if backward else 4) * w.heads * w.L * w.d * elem   # inputs read + outputs written once
    alg_flops = (22.0 if backward else 8.0) * w.heads * w.L * w.d * w.m
    achieved_tflops = alg_flops / (ms * 1e-3) / 1e12

    def roofline(nbytes, nflops, sec, alu=False):
        # alu: fp32 FMA kernels (the generic path), priced against the fp32
        # vector peak instead of the matrix cores'
        peak = FP32_VALU_PEAK_TFLOPS if alu else BF16_PEAK_TFLOPS
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = nflops / (peak * 1e12)
        if t_hbm >= t_mfma:
            a = nbytes / sec / 1e9
            return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(a / HBM_PEAK_GBS, 4)}
        a = nflops / sec / 1e12
        return {"bound": "alu" if alu else "mfma", "achieved": round(a, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(a / peak, 4)}

    _, nseg, seg = fv.plan_describe(w.B, w.H, w.L, w.d, w.m,
                                    fv.BF16 if w.dtype == "bf16" else fv.F32, w.causal)
    kernels = {}
    for name, (tot_ms, launches) in kt.items():
        kb, kf = kernel_work(name, w, nseg, seg, elem, backward)
        kernels[name] = {"avg_us": round(1e3 * tot_ms / launches, 3), "launches": launches,
                         "alg_bytes": kb, "alg_flops": kf}
    dom = max(kt, key=lambda n: kt[n][0])
    dsec = kt[dom][0] / kt[dom][1] * 1e-3
    generic = dom.startswith("g_") or dom.startswith("gb_")
    roof = roofline(kernels[dom]["alg_bytes"], kernels[dom]["alg_flops"], dsec, alu=generic)
    # (counter summaries exist for the softmax-kernel runs only)
    counted = args.kernel == "softmax" and not backward
    roof["traffic"] = measured_traffic(w.name, w.causal, dom) if counted else None
    mf = measured_counters(w.name, w.causal, dom) if counted else None
    if mf is not None:
        roof["mfma_executed_frac"] = mf
    roof["kernel"] = dom
    roof["kernel_avg_us"] = kernels[dom]["avg_us"]
    whole = roofline(alg_bytes, alg_flops, ms * 1e-3, alu=generic)
    # Secondary fractions against the measured copy ceiling (HBM-bound only).
    ceiling = copy_ceiling()
    for r in (roof, whole):
        if r["bound"] == "hbm":
            r["frac_vs_copy"] = round(r["achieved"] / ceiling["GB_s"], 4)

    out = {
        "metric": ("FAVOR+ bwd tokens*heads/s, B8 H8 L4096 d64 m256" if backward else
                   "FAVOR+ causal prefill tokens*heads/s, B8 H8 L4096 d64 m256"
                   if args.pass_ == "prefill" else
                   "FAVOR+ fwd tokens*heads/s + % of roofline, B8 H8 L4096 d64 m256"),
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
                   "causal": w.causal, "attn_kernel": args.kernel, "pass": args.pass_,
                   **({"carried_state": True} if args.carry and args.pass_ == "prefill" else {}),
                   "buffer_sets": nsets,
                   "cache": "hot" if args.cache_hot else "rotating >= 1 GiB"},
        "repeats": {"n": len(reps), "min_ms": round(reps[0], 5),
                    "median_ms": round(reps[len(reps) // 2], 5), "max_ms": round(reps[-1], 5)},
        "cache_hot_ms_per_step": round(hot, 5),
        "tflops_alg": round(achieved_tflops, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "roofline_whole_call": whole,
        "copy_ceiling": ceiling,
        "kernels": kernels,
    }
    if redraw:
        out["redraw"] = redraw
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.kernel, backward)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
