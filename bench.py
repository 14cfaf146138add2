#!/usr/bin/env python3
"""Benchmark of the NA3D forward kernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

A step is one na3d_fwd call over one batch of the synthetic workload (all
inputs resident in HBM before timing starts).  The headline workload is the
VAE-decoder tile (B=1, T=16, H=64, W=96, NH=8, HD=64, window 3x7x7).  Prints
ONE JSON line with TFLOP/s (algorithmic FLOPs = 4*B*NH*T*H*W*KT*KH*KW*HD), the
roofline of the kernel (HBM-bound at this arithmetic intensity: algorithmic
bytes = q, k, v read once + out written once = 8*HD bytes per query-head) and
the CPU oracle's throughput on a bounded sample of the same workload.

    python bench.py --copy-calibration BYTES

runs a plain device-to-device copy of BYTES bytes a few times and nothing
else: the reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
HEADLINE = "decoder_tile"
METRIC = "NA3D fwd TFLOP/s and % bf16 MFMA peak on 1 MI355X, (3,7,7)/(11,11,11)"
KERNEL_SOURCES = ("neighborhood_attention_amd/csrc/common.h",
                  "neighborhood_attention_amd/csrc/kernel_roll.hip",
                  "neighborhood_attention_amd/csrc/kernel_general.hip",
                  "neighborhood_attention_amd/csrc/na3d.cpp")
NORM_SOURCES = ("neighborhood_attention_amd/csrc/common.h",
                "neighborhood_attention_amd/csrc/kernel_rmsnorm.hip",
                "neighborhood_attention_amd/csrc/na3d.cpp")
NORM_EPS = 1e-6
WARMUP_MIN_S = 0.05  # least wall time of warm-up launches before a timed region


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--all", action="store_true",
                    help="one JSON line per workload (development use)")
    ap.add_argument("--pages-grid", action="store_true",
                    help="time the six grids of the aiter PR's Performance table at NH = 4, 8 "
                         "and 32 (one JSON line each; development use)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large-window", action="store_true",
                    help="headline run without the 11x11x11 companion measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="headline run without the full-scale, narrow and tiny companions")
    ap.add_argument("--no-fused", action="store_true",
                    help="headline run without the fused-QKV input companion measurement")
    ap.add_argument("--no-split", action="store_true",
                    help="headline run without the 2x2 query-box split companion measurement")
    ap.add_argument("--no-batch", action="store_true",
                    help="headline run without the batched decoder-tiles companion measurement")
    ap.add_argument("--no-rms-norm", action="store_true",
                    help="headline run without the RMSNorm block-norm companion measurement")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache single-launch timings (counter runs)")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the sampled parity check before timing")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    return ap.parse_args()


def sources_sha256(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, profile="na3d_fwd_roll_%s_traffic.md", sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed counter summary of this
    workload, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", profile % workload)
    if not os.path.exists(path) and "_roll_" in profile:
        path = os.path.join(ROOT, "profiles", profile.replace("_roll_", "_general_") % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not tb or sha.group(1) != sources_sha256(sources):
        return None
    return float(tb.group(1))


def warm_up(fn, warmup):
    """At least `warmup` launches and at least WARMUP_MIN_S of them: the GPU
    sits idle while the host checks parity, and its clocks take a few
    milliseconds of work to come back up (a 50-launch decoder-tile region
    measured 164 us per launch after 5 warm-up launches, 144 us after 200)."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    _WARMED[0] = n
    return n


_WARMED = [0]  # warm-up launches of the last timed region


def time_kernel(fn, steps, warmup):
    """Warm up (warm_up), then time `steps` back-to-back launches.  Returns
    (wall ms per step, kernel ms per launch from HIP events recorded on the
    stream the kernel is launched on: torch's current stream, which fn
    uses)."""
    import torch

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # no garbage-collection pass of the host process inside the timed region;
    # the collection runs before the warm-up, so the GPU goes from the
    # warm-up launches to the timed ones without an idle stretch between
    gc.collect()
    gc.disable()
    try:
        warm_up(fn, warmup)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    finally:
        gc.enable()
    return wall_ms, e0.elapsed_time(e1) / steps


def time_graph(fn, steps):
    """Kernel ms per launch with `steps` launches captured in one HIP graph and
    replayed on the current stream, timed with HIP events on that stream: the
    kernels run back to back with no host launch gaps between them, which
    shows the duration of kernels shorter than the host's launch interval
    (a launch from Python takes longer to issue than a 10-20 us kernel takes
    to run)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / steps


def per_launch_us(fn, reps, cold_bytes=0):
    """Median and minimum of single-launch kernel times (HIP events around
    each launch on the launch stream).  cold_bytes > 0: before every launch a
    buffer of that size is overwritten and the GPU drained, so the launch
    starts with the inputs evicted from L2 and the 256 MB MALL."""
    import statistics

    import torch

    stream = torch.cuda.current_stream()
    scratch = None
    if cold_bytes:
        scratch = torch.empty(cold_bytes // 4, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for i, (e0, e1) in enumerate(evs):
        if scratch is not None:
            scratch.fill_(float(i))
            torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
    return {"median": round(statistics.median(t), 2), "min": round(min(t), 2), "reps": reps}


def sampled_check(q, k, v, window, out, seed, npts=400):
    """Parity gate before timing (validate, then time): oracle vs GPU on
    sampled outputs.  Returns the errors and the host copies of the inputs."""
    import oracle
    import torch

    shape = tuple(q.shape)
    rng = np.random.default_rng(seed)
    pts = np.stack([rng.integers(0, s, npts) for s in shape[:5]], axis=1)
    idx = tuple(torch.as_tensor(pts[:, i], device=q.device) for i in range(5))
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    ref = oracle.fwd_points(qc, kc, vc, window, pts)
    got = out[idx].double().cpu().numpy()
    diff = got - ref
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    return rel, float(np.abs(diff).max()), (qc, kc, vc)


def cpu_baseline(host_inputs, window, seed, target_s):
    """Time the oracle (as it stands) on a bounded random sample of the
    workload's query-heads, sized for about target_s seconds; returns its
    TFLOP/s (same algorithmic FLOP count per query-head as the metric)."""
    import oracle

    qc, kc, vc = host_inputs
    shape = tuple(qc.shape)
    KT, KH, KW = window
    HD = shape[5]
    per_query = 4 * KT * KH * KW * HD
    total_q = int(np.prod(shape[:5]))
    rng = np.random.default_rng(seed + 17)
    threads = oracle.max_threads(0)

    def run(n):
        pts = np.stack([rng.integers(0, s, n) for s in shape[:5]], axis=1)
        t0 = time.perf_counter()
        oracle.fwd_points(qc, kc, vc, window, pts)
        return time.perf_counter() - t0

    pilot = min(2000, total_q)
    dt = run(pilot)
    n = int(min(total_q, max(pilot, pilot * target_s / max(dt, 1e-9))))
    dt = run(n)
    return {
        "value": round(n * per_query / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d random query-heads of %d (%.2f%%) of the same workload and inputs, "
                  "%.1f s of oracle time, fp64, %d OpenMP threads"
                  % (n, total_q, 100.0 * n / total_q, dt, threads),
    }


def bench_workload(name, steps, warmup, check=True, cpu=True, cpu_s=10.0, cold=True):
    import torch

    import neighborhood_attention_amd as na
    from na3d_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    q, k, v = make_inputs(w.shape, w.seed, "cuda", w.k_outlier_frac, w.k_outlier_scale)
    out = torch.empty_like(q)
    fn = lambda: na.fwd(q, k, v, w.window, out=out)
    fn()
    torch.cuda.synchronize()
    rel = mab = None
    host = None
    if check or cpu:
        rel, mab, host = sampled_check(q, k, v, w.window, out, w.seed)
        if rel > 1e-2 or mab > 5e-2:
            raise SystemExit("parity gate failed on %s: rel_l2=%.3e max_abs=%.3e"
                             % (name, rel, mab))
    wall_ms, kern_ms = time_kernel(fn, steps, warmup)
    warmed = _WARMED[0]
    graph_ms = time_graph(fn, steps)
    single = {"warm": per_launch_us(fn, steps)}
    if cold:
        single["cold"] = per_launch_us(fn, max(steps // 2, 5), cold_bytes=512 << 20)
        single["cold"]["between_launches"] = "512 MiB written, GPU drained"
    tflops = w.flops / (wall_ms * 1e-3) / 1e12
    # the roofline is that of the kernel's duration over the timed region
    # (HIP events on the launch stream); the graph replay is reported beside
    # it, since for kernels shorter than the host's launch interval the eager
    # loop includes launch gaps
    kern_s = kern_ms * 1e-3
    ai = w.flops / w.bytes
    bound = "mfma" if ai > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    if bound == "hbm":
        achieved, peak, unit = w.bytes / kern_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = w.flops / kern_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    plan = na.plan(w.shape, w.window)
    tbytes = measured_traffic(name)  # HBM bytes per launch from the counters, if current
    hashes = None
    if host is not None:
        from na3d_inputs import sha256_of
        hashes = {n_: sha256_of(t) for n_, t in zip("qkv", host)}
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "warmup_policy": "at least `warmup` launches and at least %d ms of them" % round(
            WARMUP_MIN_S * 1e3),
        "warmup_launches": warmed,
        "ms_per_step": round(wall_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name,
            "shape_BTHWNH_HD": list(w.shape),
            "window": list(w.window),
            "seed": w.seed,
            "family": "rolling" if plan["family"] == 2 else "general",
            "variant": plan["variant"],
            "tile": [plan["tile_t"], plan["tile_h"], plan["tile_w"]],
            "workgroups": plan["workgroups"],
        },
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 5),
        "effective_GBps": round(w.bytes / (wall_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            # measured HBM bytes per launch over the same launch time (GB/s):
            # comparable with `achieved` for the HBM-bound workloads
            "traffic": None if tbytes is None else round(tbytes / kern_s / 1e9, 2),
            "traffic_bytes_per_launch": tbytes,
        },
        "kernel_us": round(kern_ms * 1e3, 2),
        "kernel_us_graph": round(graph_ms * 1e3, 2),
        "per_launch_us": single,
        "parity_sampled": {"rel_l2": rel, "max_abs": mab},
        "inputs_sha256": hashes,
    }
    if cpu and host is not None:
        cb = cpu_baseline(host, w.window, w.seed, cpu_s)
        cb["cpu_model"] = cpu_model()
        cb["gpu_over_oracle"] = round(tflops / cb["value"], 1) if cb["value"] > 0 else None
        rec["cpu_baseline"] = cb
    return rec


def companion(name, steps, warmup, cold=False):
    """A further workload in the same run, reported beside the headline with
    its own roofline (parity gate first, as for the headline)."""
    rec = bench_workload(name, steps, warmup, check=True, cpu=False, cold=cold)
    return {k: rec[k] for k in ("value", "unit", "mfma_peak_frac", "ms_per_step", "kernel_us",
                                "kernel_us_graph", "per_launch_us", "roofline", "parity_sampled",
                                "inputs_sha256", "warmup_launches")} | {
        "shape_BTHWNH_HD": rec["config"]["shape_BTHWNH_HD"], "window": rec["config"]["window"],
        "family": rec["config"]["family"], "variant": rec["config"]["variant"],
        "workgroups": rec["config"]["workgroups"]}


def bench_fused(name, steps, warmup):
    """The headline workload with q, k, v read in place from one fused
    (B,T,H,W,3,NH,HD) QKV buffer through the strided entry point, against
    first copying them out to contiguous tensors (what a launcher that only
    takes contiguous inputs must do).  Returns kernel-time figures."""
    import torch

    import neighborhood_attention_amd as na
    from na3d_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    q, k, v = make_inputs(w.shape, w.seed, "cuda", w.k_outlier_frac)
    qkv = torch.stack([q, k, v], dim=4).contiguous()
    del q, k, v
    qs, ks, vs = (qkv[:, :, :, :, i] for i in range(3))
    out = torch.empty(w.shape, dtype=torch.bfloat16, device="cuda")
    ref = na.fwd(qs.contiguous(), ks.contiguous(), vs.contiguous(), w.window)
    na.fwd(qs, ks, vs, w.window, out=out)
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise SystemExit("fused-QKV output differs from the contiguous path")
    _, strided_ms = time_kernel(lambda: na.fwd(qs, ks, vs, w.window, out=out), steps, warmup)
    bufs = [torch.empty(w.shape, dtype=torch.bfloat16, device="cuda") for _ in range(3)]

    def copy_then_run():
        for dst, src in zip(bufs, (qs, ks, vs)):
            dst.copy_(src)
        na.fwd(bufs[0], bufs[1], bufs[2], w.window, out=out)

    _, copy_ms = time_kernel(copy_then_run, steps, warmup)
    return {
        "layout": "(B,T,H,W,3,NH,HD) fused QKV buffer, q/k/v as strided views",
        "value": round(w.flops / (strided_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "kernel_us_strided": round(strided_ms * 1e3, 2),
        "us_copy_to_contiguous_then_kernel": round(copy_ms * 1e3, 2),
        "bitwise_equal_to_contiguous": True,
    }


def bench_split(name, steps, warmup):
    """The headline workload's queries split into 2 x 2 boxes along H and W,
    each computed by the query-box entry point with windows in the whole grid
    (what one GPU of a spatial split runs), against one whole-grid launch."""
    import torch

    import neighborhood_attention_amd as na
    from na3d_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    B, T, H, W, NH, HD = w.shape
    q, k, v = make_inputs(w.shape, w.seed, "cuda", w.k_outlier_frac)
    whole = torch.empty_like(q)
    parts = torch.empty_like(q)
    boxes = [(0, h0, w0, T, hq, wq) for h0, hq in ((0, H // 2), (H // 2, H - H // 2))
             for w0, wq in ((0, W // 2), (W // 2, W - W // 2))]
    views = [(q[:, :, b[1]:b[1] + b[4], b[2]:b[2] + b[5]],
              parts[:, :, b[1]:b[1] + b[4], b[2]:b[2] + b[5]], b) for b in boxes]

    def run_parts():
        for qb, ob, b in views:
            na.fwd_subgrid(qb, k, v, w.window, b[:3], out=ob)

    na.fwd(q, k, v, w.window, out=whole)
    run_parts()
    torch.cuda.synchronize()
    a = whole.double()
    rel = float((parts.double() - a).norm() / a.norm())
    if rel > 2e-3:
        raise SystemExit("query-box split differs from the whole grid: rel %.3e" % rel)
    _, whole_ms = time_kernel(lambda: na.fwd(q, k, v, w.window, out=whole), steps, warmup)
    _, parts_ms = time_kernel(run_parts, steps, warmup)
    return {
        "boxes": [list(b) for b in boxes],
        "kernel_us_whole": round(whole_ms * 1e3, 2),
        "kernel_us_four_boxes": round(parts_ms * 1e3, 2),
        "rel_l2_vs_whole": rel,
    }


def bench_rms_norm(launches=400, warmup=20, check=True, cpu_s=3.0):
    """The bf16 RMSNorm block norm on its stand-in workload (24576 tokens x
    4096 channels, with weight): HBM-bound, so the figure is GB/s of
    algorithmic bytes (x read once, y written once, the weight once) against
    the 8 TB/s peak.  Parity gate first: every element of 64 random rows
    against the oracle, within the kernel's one-rounding bound.  A launch
    takes about 60 us, so the headline's step count is multiplied by 8."""
    import torch

    import neighborhood_attention_amd as na
    from na3d_inputs import NORM_WORKLOADS, make_norm_inputs
    from oracle.rmsnorm import rms_norm as oracle_rms_norm

    wl = NORM_WORKLOADS["rms_block_norm"]
    x, w = make_norm_inputs(wl.rows, wl.dim, wl.seed, "cuda")
    y = torch.empty_like(x)
    fn = lambda: na.rms_norm(x, w, NORM_EPS, out=y)
    fn()
    torch.cuda.synchronize()
    rng = np.random.default_rng(wl.seed)
    sample = np.sort(rng.choice(wl.rows, 64, replace=False))
    xs = x[torch.as_tensor(sample, device=x.device)].float().cpu().numpy()
    wn = w.float().cpu().numpy()
    worst = None
    if check:
        ref = oracle_rms_norm(xs, wn, NORM_EPS)
        got = y[torch.as_tensor(sample, device=x.device)].double().cpu().numpy()
        ratio = np.abs(got - ref) / (np.abs(ref) + 1e-30)
        worst = float(ratio.max())
        if worst > 2.0 ** -8 + 2.0 ** -14:
            raise SystemExit("parity gate failed on the RMSNorm workload: worst relative "
                             "error %.3e" % worst)
    _, kern_ms = time_kernel(fn, launches, warmup)
    warmed = _WARMED[0]
    kern_s = kern_ms * 1e-3
    tbytes = measured_traffic(wl.name, "rms_norm_%s_traffic.md", NORM_SOURCES)
    gbs = wl.bytes / kern_s / 1e9
    # CPU baseline: the oracle (numpy, one thread) on a bounded number of rows,
    # GB/s of the same algorithmic bytes per row
    n = 256
    t0 = time.perf_counter()
    oracle_rms_norm(xs.repeat(n // 64, axis=0), wn, NORM_EPS)
    dt = time.perf_counter() - t0
    n = int(min(wl.rows, max(n, n * cpu_s / max(dt, 1e-9))))
    xb = np.resize(xs, (n, wl.dim))
    t0 = time.perf_counter()
    oracle_rms_norm(xb, wn, NORM_EPS)
    dt = time.perf_counter() - t0
    per_row = wl.bytes / wl.rows
    return {
        "workload": wl.name, "rows": wl.rows, "dim": wl.dim, "weight": True, "eps": NORM_EPS,
        "launches": launches, "warmup_launches": warmed, "kernel_us": round(kern_ms * 1e3, 2),
        "value": round(gbs, 1), "unit": "GB/s",
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": None if tbytes is None else round(tbytes / kern_s / 1e9, 1),
            "traffic_bytes_per_launch": tbytes,
        },
        "parity_sampled": {"rows": 64, "worst_rel_err": worst},
        "cpu_baseline": {
            "value": round(n * per_row / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d rows (copies of 64 sampled rows) of %d, %.1f s of numpy fp64 time"
                      % (n, wl.rows, dt),
        },
    }


def bench_batch(steps, warmup):
    """A corner of a decoder tile grid, 2 x 3 tiles with narrow right and
    bottom edges ((16,64,96) x 2, (16,64,7) x 2, (16,32,96), (16,32,7); NH=8,
    HD=64, window 3x7x7), run as one batch (na3d_fwd_batch: one launch)
    against one na3d_fwd launch per tile back to back.  Every batched output
    is first checked bitwise against the same tile run alone with the
    batch's instantiation."""
    import torch

    import neighborhood_attention_amd as na
    from na3d_inputs import make_inputs

    NH, HD, ks = 8, 64, (3, 7, 7)
    dims = [(1, 16, 64, 96)] * 2 + [(1, 16, 64, 7)] * 2 + [(1, 16, 32, 96), (1, 16, 32, 7)]
    qkv = [make_inputs(d + (NH, HD), 40 + i, "cuda") for i, d in enumerate(dims)]
    outs = [torch.empty_like(t[0]) for t in qkv]
    plan = na.plan_batch(dims, NH, HD, ks)
    na.fwd_batch(qkv, ks, outs=outs)
    for (q, k, v), o in zip(qkv, outs):
        if not torch.equal(o, na.fwd(q, k, v, ks, config=(2, plan["variant"], 0))):
            raise SystemExit("batched tile differs from the same tile run alone")
    torch.cuda.synchronize()
    solo = [torch.empty_like(t[0]) for t in qkv]

    def separate():
        for (q, k, v), o in zip(qkv, solo):
            na.fwd(q, k, v, ks, out=o)

    _, batch_ms = time_kernel(lambda: na.fwd_batch(qkv, ks, outs=outs), steps, warmup)
    _, sep_ms = time_kernel(separate, steps, warmup)
    flops = sum(4 * d[0] * d[1] * d[2] * d[3] * NH * ks[0] * ks[1] * ks[2] * HD for d in dims)
    return {
        "tiles": [list(d) for d in dims], "NH": NH, "HD": HD, "window": list(ks),
        "launches": plan["launches"], "variant": plan["variant"],
        "kernel_us_batched": round(batch_ms * 1e3, 2),
        "kernel_us_one_launch_per_tile": round(sep_ms * 1e3, 2),
        "value": round(flops / (batch_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "bitwise_equal_to_tiles_alone": True,
    }


def copy_bandwidth(nbytes=1 << 30, reps=20):
    """A plain device-to-device copy (torch's), GB/s counting the bytes read
    and written: the streaming rate a simple kernel reaches on this GPU,
    beside the 8 TB/s specification."""
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    _, ms = time_kernel(lambda: dst.copy_(src), reps, 3)
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def gemm_tflops(n=8192, reps=20):
    """A plain bf16 GEMM (torch.matmul, i.e. hipBLASLt) of n x n x n: the MFMA
    rate a tuned library kernel reaches on this GPU, beside the 2.5 PFLOP/s
    specification."""
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    _, ms = time_kernel(lambda: torch.matmul(a, b, out=c), reps, 3)
    return round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_clocks():
    """Shader and memory clocks of the GPU as the amdgpu driver reports them
    in sysfs (read as plain files: no other program is started from this
    GPU-using process): the DPM levels with the current one marked, and
    the hwmon frequency readings (MHz); sampled right after a timed region,
    so the GPU is still clocked up.  Empty where the files are not there."""
    import glob

    out = {"source": "sysfs (amdgpu)"}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        found = {}
        for name, key in (("pp_dpm_sclk", "sclk_levels"), ("pp_dpm_mclk", "mclk_levels")):
            try:
                with open(os.path.join(dev, name)) as f:
                    txt = f.read()
            except OSError:
                continue
            levels = [ln.strip() for ln in txt.splitlines() if ln.strip()]
            found[key] = levels[:16]
            cur = [ln for ln in levels if ln.endswith("*")]
            if cur:
                m = re.search(r"(\d+)\s*[Mm]hz", cur[0])
                if m:
                    found[key.replace("levels", "cur_MHz")] = int(m.group(1))
        for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
            for i in (1, 2):
                try:
                    with open(os.path.join(hw, "freq%d_label" % i)) as f:
                        label = f.read().strip()
                    with open(os.path.join(hw, "freq%d_input" % i)) as f:
                        found["%s_MHz" % label] = int(f.read().strip()) // 1000000
                except (OSError, ValueError):
                    continue
        if found:
            out[os.path.basename(os.path.dirname(dev))] = found
            break
    return out


def provenance():
    import torch

    return {
        "torch": torch.__version__, "hip": torch.version.hip,
        "gpu": torch.cuda.get_device_name(0),
        "cpu_model": cpu_model(), "host_threads": len(os.sched_getaffinity(0)),
    }


# The grids of the aiter PR page's Performance table (bf16, B=1, HD=64; the
# head count per row is not stated), with the page's gfx950 (MI350X) kernel
# times in microseconds, which include a v.contiguous() copy.
PAGES_GRID = (
    ((18, 32, 48), (3, 7, 7), 1249),
    ((36, 64, 96), (3, 5, 5), 1910),
    ((40, 96, 96), (3, 5, 5), 3319),
    ((16, 80, 32), (11, 11, 11), 1153),
    ((79, 192, 192), (11, 11, 11), 99143),
    ((4, 8, 128), (3, 5, 27), 40),
)


def bench_pages_grid(steps, warmup):
    """Our kernel on the page's benchmark grids at NH = 4, 8, 32.  Yields one
    record per (grid, NH)."""
    import torch

    import neighborhood_attention_amd as na
    from na3d_inputs import make_inputs

    for (T, H, W), ks, page_us in PAGES_GRID:
        for NH in (4, 8, 32):
            shape = (1, T, H, W, NH, 64)
            q, k, v = make_inputs(shape, 60 + T + NH, "cuda")
            out = torch.empty_like(q)
            fn = lambda: na.fwd(q, k, v, ks, out=out)
            n = max(3, min(steps, int(2e5 / max(page_us, 1))))
            _, ms = time_kernel(fn, n, min(warmup, n))
            flops = 4 * NH * T * H * W * ks[0] * ks[1] * ks[2] * 64
            plan = na.plan(shape, ks)
            yield {"grid_THW": [T, H, W], "window": list(ks), "NH": NH, "HD": 64,
                   "kernel_us": round(ms * 1e3, 2), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
                   "page_gfx950_us": page_us, "variant": plan["variant"], "launches": n}
            del q, k, v, out
            torch.cuda.empty_cache()


def copy_calibration(nbytes):
    """A plain device copy of a known size, for scaling memory counters."""
    import torch

    n = max(nbytes // 2, 1)
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 2 * n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the NA3D path here has no multi-GPU "
              "code (--gpus %d requested); run with --gpus 1" % args.gpus, file=sys.stderr)
        return 2
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    if args.pages_grid:
        for rec in bench_pages_grid(args.steps, args.warmup):
            print(json.dumps(rec), flush=True)
        return 0
    if args.all:
        from na3d_inputs import WORKLOADS
        for name in WORKLOADS:
            rec = bench_workload(name, args.steps, args.warmup, check=not args.no_check,
                                 cpu=False)
            print(json.dumps(rec), flush=True)
        return 0
    rec = bench_workload(args.workload, args.steps, args.warmup, check=not args.no_check,
                         cpu=not args.no_cpu_baseline, cpu_s=args.cpu_seconds,
                         cold=not args.no_cold)
    clocks = gpu_clocks()  # right after the headline's timed launches
    if args.workload == HEADLINE and not args.no_large_window:
        # the metric also names the 11x11x11 window: report it beside the headline
        lw = bench_workload("large_window", args.steps, args.warmup, check=not args.no_check,
                            cpu=False, cold=not args.no_cold)
        rec["large_window_11x11x11"] = {
            "value": lw["value"], "unit": "TFLOP/s", "mfma_peak_frac": lw["mfma_peak_frac"],
            "ms_per_step": lw["ms_per_step"], "kernel_us": lw["kernel_us"],
            "kernel_us_graph": lw["kernel_us_graph"],
            "per_launch_us": lw["per_launch_us"],
            "roofline": lw["roofline"], "parity_sampled": lw["parity_sampled"],
            "inputs_sha256": lw["inputs_sha256"], "variant": lw["config"]["variant"],
            "workgroups": lw["config"]["workgroups"], "warmup_launches": lw["warmup_launches"]}
        # the pages' anisotropic wide-window benchmark grid, (3,5,27)
        ww = bench_workload("wide_w27", args.steps, args.warmup, check=not args.no_check,
                            cpu=False, cold=not args.no_cold)
        rec["wide_window_3x5x27"] = {
            "shape_BTHWNH_HD": ww["config"]["shape_BTHWNH_HD"], "value": ww["value"],
            "unit": "TFLOP/s", "kernel_us": ww["kernel_us"],
            "kernel_us_graph": ww["kernel_us_graph"], "roofline": ww["roofline"],
            "parity_sampled": ww["parity_sampled"], "variant": ww["config"]["variant"],
            "warmup_launches": ww["warmup_launches"]}
        # a window wider than 33 along W (the shapes the pages' kernel refused)
        rec["wide_window_3x5x41"] = companion("wide_w41", args.steps, args.warmup)
        # a 19x19x19 window: the four-group rolling instantiation at head dim
        # 64, and the slowest path, the general family, at head dim 128
        # (whose halo no rolling instantiation's LDS holds; ~2 ms a launch)
        rec["window_19x19x19"] = companion("window_19", max(3, min(args.steps, 10)),
                                           min(args.warmup, 2))
        rec["general_family_19x19x19"] = companion("window_19_hd128", max(3, min(args.steps, 10)),
                                                   min(args.warmup, 2))
    if args.workload == HEADLINE and not args.no_configs:
        # the remaining workloads of the metric's configuration list, each with
        # its own roofline: full scale (HD 128, x8 key outliers; fewer
        # launches: ~5 ms each), the two narrow edge tiles and the tiny grid
        rec["full_scale"] = companion("full_scale", max(5, min(args.steps, 20)),
                                      min(args.warmup, 3))
        for nm in ("narrow_w7", "narrow_w5", "tiny"):
            rec[nm] = companion(nm, args.steps, args.warmup)
    if args.workload == HEADLINE and not args.no_fused:
        rec["fused_qkv_inputs"] = bench_fused(args.workload, args.steps, args.warmup)
    if args.workload == HEADLINE and not args.no_split:
        rec["query_box_split_2x2"] = bench_split(args.workload, args.steps, args.warmup)
    if args.workload == HEADLINE:
        rec["measured_copy_GBps"] = copy_bandwidth()
        rec["measured_gemm_TFLOPs"] = gemm_tflops()
        # roofline fractions against what a device copy and a library GEMM
        # reach here, beside the specification peaks
        meas = {"hbm": rec["measured_copy_GBps"], "mfma": rec["measured_gemm_TFLOPs"]}
        for sub in [rec] + [rec[k] for k in ("large_window_11x11x11", "wide_window_3x5x27",
                                             "wide_window_3x5x41", "window_19x19x19",
                                             "general_family_19x19x19",
                                             "full_scale", "narrow_w7", "narrow_w5", "tiny")
                            if k in rec]:
            rf = sub["roofline"]
            rf["measured_peak"] = meas[rf["bound"]]
            rf["frac_of_measured_peak"] = round(rf["achieved"] / meas[rf["bound"]], 4)
        rec["provenance"] = provenance()
        rec["provenance"]["clocks"] = clocks
    if args.workload == HEADLINE and not args.no_batch:
        rec["decoder_tiles_batched"] = bench_batch(args.steps, args.warmup)
    if args.workload == HEADLINE and not args.no_rms_norm:
        rec["rms_norm_block_norm"] = bench_rms_norm(8 * args.steps, 4 * args.warmup,
                                                    check=not args.no_check,
                                                    cpu_s=0.0 if args.no_cpu_baseline else 3.0)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
