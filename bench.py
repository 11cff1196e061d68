#!/usr/bin/env python3
"""Benchmark of row-wise softmax with the online normalizer on one MI355X.

Workload (the benchmark's headline configuration): 4096 rows x 32000 columns of
fp32 LM-logit rows, 2*N(0,1) with 0.1% of entries at +-80 and 0.01% at -inf
(seeded synthetic, ``workloads.config(2)``), fp32 output.  A step is one
``os_softmax_forward`` over the whole batch: the fold into (m, d), the merge,
and the normalising pass.

Printed: one JSON line.  ``value`` is the effective HBM bandwidth, algorithmic
bytes (one read of the input + one write of the output) per second of wall
time over the timed steps; ``rows_per_s`` the same in rows.  ``roofline``
prices the dominant kernel against the 8 TB/s HBM peak using its average
duration from HIP events recorded on the launch stream; ``traffic`` is the
HBM bytes per launch from rocprofv3 counters (``profiles/``), or null when the
kernels changed since the counters were taken.  ``cpu_baseline`` is the CPU
oracle timed on this host.  Comparison legs on the same input: the three-pass
safe-softmax baseline, the unshifted two-pass baseline, the streaming two-pass
kernel, and two copies.  ``exp_rate`` is the measured rate of the hardware
exponential (the arithmetic ceiling beside HBM).  ``workloads`` times all five
workloads in the launch configuration the parity tests check: kernel time,
fraction of the HBM peak, rows/s, the same from a flushed cache, the section 5
baselines, the fused top-K against its unfused pipelines, and the CPU oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
CUS = 256           # MI355X compute units
CLOCK_HZ = 2.4e9    # MI355X peak engine clock
KERNEL_SOURCES = ["online_normalizer_amd/csrc/os_kernels.hpp", "online_normalizer_amd/csrc/os_device.hpp",
                  "online_normalizer_amd/csrc/os_abi.hip"]
COUNTERS_FILE = "profiles/counters_softmax_fwd_4096x32000_f32.txt"
WORKLOAD = 2


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(launch_bytes_alg: float):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, COUNTERS_FILE)
    if not os.path.exists(path):
        return None, "no counter summary"
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernels changed since the counters were taken"
    try:
        fetch = float(vals["fetch_kib_per_dispatch"]) * 1024 * float(vals["fetch_scale"])
        write = float(vals["write_kib_per_dispatch"]) * 1024 * float(vals["write_scale"])
    except (KeyError, ValueError):
        return None, "counter summary incomplete"
    return fetch + write, None


def time_graph(fn, steps: int, warmup: int, stream, replays: int = 1):
    """Capture `steps` calls of fn() in one HIP graph and time `replays`
    replays of it, each bracketed by torch.cuda.synchronize().

    Before the timed replays: `warmup` eager calls, then two untimed replays
    (the first uploads the graph; the second runs right before the timed ones,
    so that the GPU is not idle when they start).  Returns (wall seconds,
    average seconds per launch) of the replay whose average launch is the
    median, and the list of every replay's average launch."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fn()
    graph.replay()  # uploads the graph
    graph.replay()
    torch.cuda.synchronize()
    runs = []
    for _ in range(replays):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        runs.append((wall, start.elapsed_time(end) * 1e-3 / steps))
    order = sorted(range(len(runs)), key=lambda r: runs[r][1])
    wall, avg = runs[order[len(order) // 2]]
    return wall, avg, [a for _, a in runs]


def time_launches(fn, steps: int, warmup: int, stream):
    """Run fn() warmup+steps times back to back; HIP events around each timed launch."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        starts[k].record(stream)
        fn()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]
    return wall, per


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_times(fn, reps: int):
    """Wall seconds of `reps` calls of fn() (the oracle), and their median."""
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2], times


def cpu_baseline(x, bytes_per_row: float, reps: int = 3):
    """The oracle, as it stands (three-pass safe softmax in double), on every
    host core the process may use: the median wall time of `reps` passes over
    the whole workload."""
    import oracle
    orc = oracle.load()
    cores = len(os.sched_getaffinity(0))
    rows = x.shape[0]
    med, _ = oracle_times(lambda: orc.softmax(x, threads=cores), reps)
    return {
        "value": round(rows * bytes_per_row / med / 1e9, 3),
        "unit": "GB/s",
        "rows_per_s": round(rows / med, 1),
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"the whole workload, {rows} rows x {x.shape[1]} cols (3-pass safe softmax in double, "
                  f"std::thread over rows): median of {reps} passes, {med:.3f} s wall each",
    }


def exp_rate(ons, stream):
    """Measured rate of the hardware exponential: 2048 workgroups (8 waves per
    SIMD), 2048 rounds of one exponential + one fused multiply-add per chain."""
    import torch
    wgs, iters = 2048, 2048
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    res = {}
    for chains, name in ((8, "independent"), (1, "dependent")):
        _, avg, _ = time_graph(lambda: ons.os_bench_exp(out, wgs, iters, chains), 5, 2, stream, replays=3)
        rate = wgs * 256 * iters * chains / avg
        res[name] = {"Gexp_per_s": round(rate / 1e9, 1),
                     "per_CU_per_clock": round(rate / (CUS * CLOCK_HZ), 2), "us": round(avg * 1e6, 2)}
    return res


def flushed_us(fn, stream, scratch, reps: int = 10):
    """Median single launch with L2 and the Infinity Cache flushed first (a
    1 GiB fill runs before each launch, outside the HIP events)."""
    import torch
    times = []
    for _ in range(reps):
        scratch.zero_()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) * 1e-3)
    return sorted(times)[len(times) // 2] * 1e6


def per_workload(ons, stream, exp_per_s: float, x2=None, y2=None):
    """Every workload in the launch configuration the benchmark times: kernel
    time (median of 3 graph replays of 20 launches), bandwidth on the
    algorithmic bytes as a fraction of the 8 TB/s peak, rows/s, the same with
    caches flushed, the [OS] section 5 baselines on the same input (3-pass
    safe, unshifted 2-pass), and the CPU oracle on the whole workload (median
    of 3 passes; workload 1: of 100, plus one thread)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    orc = oracle.load()
    cores = len(os.sched_getaffinity(0))
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB

    def gus(fn, reps=20):
        _, avg, _ = time_graph(fn, reps, 3, stream, replays=3)
        return avg * 1e6

    table = {}
    for n in (1, 2, 3, 4):
        if n == 2 and x2 is not None:
            xh, x, y = None, x2, y2
        else:
            xh = workloads.config(n)
            x = (torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16) if xh.dtype == np.uint16
                 else torch.from_numpy(xh)).cuda()
            y = torch.empty_like(x)
        rows, cols = x.shape
        nb = rows * cols * x.element_size() * 2
        t = gus(lambda: ons.os_softmax_forward(x, out=y), 200 if n == 1 else 20)
        tf = flushed_us(lambda: ons.os_softmax_forward(x, out=y), stream, scratch)
        ts = gus(lambda: ons.safe_softmax_forward(x, out=y))
        tn = gus(lambda: ons.naive_softmax_forward(x, out=y))
        e = {"rows": rows, "cols": cols, "dtype": str(x.dtype).replace("torch.", ""),
             "algorithmic_bytes": nb, "kernel_us": round(t, 2), "GBs": round(nb / t / 1e3, 1),
             "frac": round(nb / t / 1e3 / PEAK_HBM_GBS, 4), "rows_per_s": round(rows / t * 1e6, 1),
             "flushed_us": round(tf, 2), "flushed_frac": round(nb / tf / 1e3 / PEAK_HBM_GBS, 4),
             "safe_3pass_us": round(ts, 2), "naive_2pass_us": round(tn, 2),
             "speedup_vs_safe_3pass": round(ts / t, 3)}
        if xh is None:
            xh = x.cpu().numpy()
        if n == 1:
            med, _ = oracle_times(lambda: orc.softmax(xh, threads=cores), 100)
            med1, _ = oracle_times(lambda: orc.softmax(xh, threads=1), 100)
            e["cpu_oracle"] = {"s": round(med, 6), "s_one_thread": round(med1, 6), "cores": cores,
                               "rows_per_s": round(rows / med, 1), "GBs": round(nb / med / 1e9, 3)}
        else:
            med, _ = oracle_times(lambda: orc.softmax(xh, threads=cores), 3)
            e["cpu_oracle"] = {"s": round(med, 4), "cores": cores, "rows_per_s": round(rows / med, 1),
                               "GBs": round(nb / med / 1e9, 3)}
        table[str(n)] = e
        del x, y, xh
    # workload 5: the fused top-K, its unfused pipelines, and the same logits in bf16
    xh = workloads.config(5)
    K = workloads.TOPK_K
    x = torch.from_numpy(xh).cuda()
    rows, cols = x.shape
    nb = rows * cols * 4 + rows * K * 8
    t = gus(lambda: ons.os_softmax_topk(x, K), 200)
    tf = flushed_us(lambda: ons.os_softmax_topk(x, K), stream, scratch)
    yt = torch.empty_like(x)
    legs = {}
    for name, fwd in (("unfused_online", ons.os_softmax_forward), ("unfused_safe", ons.safe_softmax_forward),
                      ("unfused_naive", ons.naive_softmax_forward)):
        def pipeline(fwd=fwd):
            fwd(x, out=yt)
            ons.os_topk_select(yt, K)
        tu = gus(pipeline, 50)
        tuf = flushed_us(pipeline, stream, scratch)
        legs[name] = {"us": round(tu, 2), "fused_speedup": round(tu / t, 2), "flushed_us": round(tuf, 2),
                      "fused_speedup_flushed": round(tuf / tf, 2)}
    tsel = gus(lambda: ons.os_topk_select(x, K), 200)
    # the read-only reference over the same bytes: the ceiling of a kernel
    # that only reads this much
    sink = torch.empty(4 * 2048, dtype=torch.float32, device="cuda")
    trd = gus(lambda: ons.os_device_read(x, sink), 200)
    trdf = flushed_us(lambda: ons.os_device_read(x, sink), stream, scratch)
    xb = x.to(torch.bfloat16)
    nb16 = rows * cols * 2 + rows * K * 8
    tb = gus(lambda: ons.os_softmax_topk(xb, K), 200)
    tbf = flushed_us(lambda: ons.os_softmax_topk(xb, K), stream, scratch)
    floor_b = max(nb16 / PEAK_HBM_GBS / 1e3, rows * cols / exp_per_s * 1e6)  # us
    med, _ = oracle_times(lambda: orc.topk(xh, K, threads=cores), 3)
    table["5"] = {"rows": rows, "cols": cols, "dtype": "float32", "K": K, "algorithmic_bytes": nb,
                  "kernel_us": round(t, 2), "GBs": round(nb / t / 1e3, 1),
                  "frac": round(nb / t / 1e3 / PEAK_HBM_GBS, 4), "rows_per_s": round(rows / t * 1e6, 1),
                  "flushed_us": round(tf, 2), "flushed_frac": round(nb / tf / 1e3 / PEAK_HBM_GBS, 4),
                  "select_only_us": round(tsel, 2),
                  "read_only_reference": {"us": round(trd, 2), "flushed_us": round(trdf, 2),
                                          "frac_of_it": round(trd / t, 4), "flushed_frac_of_it": round(trdf / tf, 4)},
                  **legs,
                  "bf16": {"kernel_us": round(tb, 2), "algorithmic_bytes": nb16,
                           "frac": round(nb16 / tb / 1e3 / PEAK_HBM_GBS, 4), "flushed_us": round(tbf, 2),
                           "flushed_frac": round(nb16 / tbf / 1e3 / PEAK_HBM_GBS, 4),
                           "floor_us_max_hbm_exp": round(floor_b, 2), "frac_vs_max_hbm_exp": round(floor_b / tb, 4)},
                  "cpu_oracle": {"s": round(med, 4), "cores": cores, "rows_per_s": round(rows / med, 1)}}
    del x, xb, yt
    table["attention"] = attention_entry(ons, stream, gus, scratch)
    del scratch
    return table


def attention_entry(ons, stream, gus, scratch):
    """The attention forward on the online normalizer (NEXT to the row
    softmax: the (m, l, o~) state carried through Q K^T and P V on the matrix
    cores), on workload 3's shape taken as attention: 256 heads x 2048 x 128,
    bf16, full and causal.  FLOPs are the two products' 4 d per visible
    (query, key) pair; the roofline is the 2.5 PFLOP/s dense bf16 peak.  The
    CPU oracle is timed on 8 of the 256 heads."""
    import math

    import numpy as np
    import torch

    import oracle
    import workloads

    q, k, v = workloads.attention_workload()
    H, N, D = q.shape
    dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.empty_like(qd)
    entry = {"heads": H, "seq": N, "head_dim": D, "dtype": "bf16", "peak_TFLOPs": PEAK_BF16_TFLOPS}
    for causal in (False, True):
        pairs = N * (N + 1) // 2 if causal else N * N
        flops = 4.0 * D * pairs * H
        t = gus(lambda: ons.os_attention_forward(qd, kd, vd, causal=causal, out=o), 10)
        tf = flushed_us(lambda: ons.os_attention_forward(qd, kd, vd, causal=causal, out=o), stream, scratch, 5)
        entry["causal" if causal else "full"] = {
            "flops": flops, "kernel_us": round(t, 2), "TFLOPs": round(flops / t / 1e6, 1),
            "frac": round(flops / t / 1e6 / PEAK_BF16_TFLOPS, 4), "flushed_us": round(tf, 2)}
    orc = oracle.load()
    cores = len(os.sched_getaffinity(0))
    hs = 8
    med, _ = oracle_times(lambda: orc.attention(q[:hs], k[:hs], v[:hs], 1.0 / math.sqrt(D), threads=cores), 3)
    entry["cpu_oracle"] = {"s_for_8_heads": round(med, 3), "cores": cores,
                           "TFLOPs": round(4.0 * D * N * N * hs / med / 1e12, 4)}
    del qd, kd, vd, o
    return entry


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replays", type=int, default=5,
                    help="timed replays of the K-step graph; the median one is reported")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as individual launches instead of HIP graph replays")
    ap.add_argument("--no-compare", action="store_true", help="skip the comparison legs")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload section")
    ap.add_argument("--all-configs", metavar="FILE", default=None,
                    help="also time the extended table (every workload, split, unaligned and router cases) "
                         "and write it to FILE as JSON")
    ap.add_argument("--perf-map", metavar="FILE", default=None,
                    help="also time the forward over row lengths from 64 to 2^20 (16-byte aligned and not, "
                         "fp32 and bf16) and the top-K over batches, row lengths and K; write a text table to FILE")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(rows are independent: each GPU would run the same kernel on its own share of rows)",
              file=sys.stderr)
        return 2

    import torch

    import online_normalizer_amd as ons
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    x_host = workloads.config(WORKLOAD)
    rows, cols = x_host.shape
    x = torch.from_numpy(x_host).to(dev)
    y = torch.empty_like(x)
    bytes_alg = rows * cols * (4 + 4)  # one read of the input, one write of the output

    step = lambda: ons.os_softmax_forward(x, out=y)  # noqa: E731
    # per-launch kernel time of eager launches (HIP events around each launch)
    _, per = time_launches(step, args.steps, args.warmup, stream)
    eager_us = sorted(per)[len(per) // 2] * 1e6
    if args.eager:
        wall, per = time_launches(step, args.steps, args.warmup, stream)
        avg = sum(per) / len(per)
        replay_us = None
    else:
        wall, avg, reps = time_graph(step, args.steps, args.warmup, stream, replays=args.replays)
        replay_us = [round(a * 1e6, 2) for a in reps]
    value = bytes_alg * args.steps / wall / 1e9
    achieved = bytes_alg / avg / 1e9
    traffic, traffic_note = load_traffic(bytes_alg)
    lanes, vecs = ons.os_forward_plan(cols)

    out = {
        "metric": "achieved HBM GB/s and rows/s for 2-pass online softmax; % of MI355X HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"LM-logit row softmax, {rows} rows x {cols} cols fp32 -> fp32, "
                               "2*N(0,1) with 0.1% +-80 and 0.01% -inf (seed 1002)",
                   "rows": rows, "cols": cols, "kernel": f"register-resident, {lanes} lanes x {vecs} "
                                                         "16-byte vectors per row"},
        "rows_per_s": round(rows * args.steps / wall, 1),
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel_us": round(avg * 1e6, 2),
            "algorithmic_bytes": bytes_alg,
        },
        "timing": ("K steps as individual launches, HIP events around each" if args.eager else
                   f"K steps captured in one HIP graph, replayed twice untimed, then {args.replays} timed "
                   "replays (each bracketed by synchronize, HIP events on the launch stream); the replay "
                   "with the median average launch is reported"),
        "replays_kernel_us": replay_us,
        "kernel_us_eager_median": round(eager_us, 2),
    }
    if traffic_note:
        out["roofline"]["traffic_note"] = traffic_note

    if not args.no_compare:
        legs = {}
        for name, fn in (("safe_3pass", lambda: ons.safe_softmax_forward(x, out=y)),
                         ("naive_2pass", lambda: ons.naive_softmax_forward(x, out=y)),
                         ("online_stream_2pass", lambda: ons.os_softmax_forward_tuned(x, 0, 0, 0, out=y))):
            _, a, _ = time_graph(fn, 20, 3, stream, replays=3)
            legs[name] = {"kernel_us": round(a * 1e6, 2), "effective_GBs": round(bytes_alg / a / 1e9, 2)}
        _, ac, _ = time_graph(lambda: ons.os_device_copy(x, y), 20, 3, stream, replays=3)
        legs["copy"] = {"kernel_us": round(ac * 1e6, 2), "GBs": round(bytes_alg / ac / 1e9, 2)}
        # the same copy with the forward's own access pattern (one 1024-lane
        # workgroup per 128 KB row, all loads before the stores)
        _, ar, _ = time_graph(lambda: ons.os_device_copy_rows(x, y), 20, 3, stream, replays=3)
        legs["copy_row_pattern"] = {"kernel_us": round(ar * 1e6, 2), "GBs": round(bytes_alg / ar / 1e9, 2)}
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        af = flushed_us(step, stream, scratch)
        del scratch
        legs["online_flushed"] = {"kernel_us": round(af, 2), "effective_GBs": round(bytes_alg / af / 1e3, 2)}
        legs["speedup_vs_safe_3pass"] = round(legs["safe_3pass"]["kernel_us"] / (avg * 1e6), 3)
        legs["speedup_vs_naive_2pass"] = round(legs["naive_2pass"]["kernel_us"] / (avg * 1e6), 3)
        legs["pct_of_copy"] = round(100.0 * ac / avg, 2)
        legs["pct_of_row_pattern_copy"] = round(100.0 * ar / avg, 2)
        out["compare"] = legs

    ex = exp_rate(ons, stream)
    out["exp_rate"] = ex
    if not args.no_workloads:
        out["workloads"] = per_workload(ons, stream, ex["independent"]["Gexp_per_s"] * 1e9, x, y)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_host, cols * 8)

    if args.all_configs:
        with open(args.all_configs, "w") as f:
            json.dump(all_configs(ons, stream), f, indent=1)
    if args.perf_map:
        with open(args.perf_map, "w") as f:
            f.write(perf_map(ons, stream))

    print(json.dumps(out), flush=True)
    return 0


def perf_map(ons, stream) -> str:
    """The performance envelope beyond the five workloads: the forward over
    row lengths (about 256 MiB of input per launch, or 256 rows where rows are
    longer), and the fused top-K over batches, row lengths and K.  Inputs are
    N(0, 3^2) from a seeded generator.  Times are the average launch of a
    captured HIP graph of 20 launches; GB/s counts the algorithmic bytes (in +
    out for the forward, in for the top-K)."""
    import torch

    def graph_us(fn):
        _, avg, _ = time_graph(fn, 20, 3, stream)
        return avg * 1e6

    lines = ["# Forward and fused top-K across shapes on MI355X (gfx950), from:",
             "#   python bench.py --perf-map <file>",
             "# us = average launch of a captured HIP graph of 20 launches; % = of the 8 TB/s HBM peak;",
             "# 'odd' rows are not 16-byte aligned (row bytes not a multiple of 16)",
             "",
             f"{'forward':>8s} {'dtype':>8s} {'rows':>9s} {'cols':>8s} {'shape':>9s} {'us':>10s} {'GB/s':>8s} {'%':>6s}"]
    gen = torch.Generator("cuda").manual_seed(1234)
    for dt in (torch.float32, torch.bfloat16):
        es = 2 if dt == torch.bfloat16 else 4
        for cols in (64, 128, 127, 512, 1000, 1024, 2047, 2048, 4096, 8191, 8192, 16384, 32000, 32001,
                     50257, 65536, 100000, 128256, 131072, 262144, 1 << 20):
            rows = max(256, (256 << 20) // (cols * es))
            x = (torch.randn(rows, cols, device="cuda", generator=gen) * 3).to(dt)
            y = torch.empty_like(x)
            t = graph_us(lambda: ons.os_softmax_forward(x, out=y))
            nb = 2 * rows * cols * es
            lanes, vecs = ons.os_forward_plan(cols, dt)
            shape = f"{lanes}x{vecs}" if lanes else ("hybrid" if cols <= 262144 else "stream")
            odd = " odd" if (cols * es) % 16 else ""
            lines.append(f"{'':>8s} {str(dt)[6:]:>8s} {rows:>9d} {cols:>8d} {shape:>9s} {t:>10.2f} "
                         f"{nb / t / 1e3:>8.1f} {100 * nb / t / 1e3 / PEAK_HBM_GBS:>6.1f}{odd}")
            del x, y
    lines += ["", f"{'top-K':>8s} {'dtype':>8s} {'rows':>9s} {'cols':>8s} {'K':>3s} {'splits':>6s} {'us':>10s} "
                  f"{'GB/s':>8s} {'%':>6s}"]
    for dt in (torch.float32, torch.bfloat16):
        es = 2 if dt == torch.bfloat16 else 4
        for rows, cols in ((65536, 16), (65536, 64), (65536, 128), (1024, 256), (16384, 256), (65536, 256),
                           (16384, 512), (4096, 2048), (2048, 8192), (1024, 32000), (4096, 32000), (256, 50257),
                           (16, 128256), (64, 128256), (256, 128256), (1024, 128256), (16, 1 << 20)):
            x = (torch.randn(rows, cols, device="cuda", generator=gen) * 3).to(dt)
            for K in (1, 8, 32):
                if K > cols:
                    continue
                S = ons.os_topk_plan(rows, cols, K)
                ws = None
                if S > 1:
                    ws = torch.empty(ons.os_softmax_topk_workspace_bytes(rows, K, S), dtype=torch.uint8,
                                     device="cuda")
                t = graph_us(lambda: ons.os_softmax_topk_ex(x, K, S, ws))
                nb = rows * cols * es + rows * K * 8
                lines.append(f"{'':>8s} {str(dt)[6:]:>8s} {rows:>9d} {cols:>8d} {K:>3d} {S:>6d} {t:>10.2f} "
                             f"{nb / t / 1e3:>8.1f} {100 * nb / t / 1e3 / PEAK_HBM_GBS:>6.1f}")
            del x
    return "\n".join(lines) + "\n"


def all_configs(ons, stream):
    """Per-workload kernel times: the average launch of a captured HIP graph of
    back-to-back launches ("us"), and the median of single launches with HIP
    events around each ("us_eager", which adds the launch ramp)."""

    def measure(fn, reps):
        _, avg, _ = time_graph(fn, reps, 5, stream)
        _, per = time_launches(fn, reps, 5, stream)
        return avg, sorted(per)[len(per) // 2]

    def flushed(fn, reps=15):
        """Median single launch with L2 and the Infinity Cache flushed first
        (a 1 GiB fill runs before each launch, outside the events)."""
        times = []
        for _ in range(reps):
            scratch.zero_()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            torch.cuda.synchronize()
            times.append(s.elapsed_time(e) * 1e-3)
        return sorted(times)[len(times) // 2]

    import numpy as np
    import torch

    import workloads

    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    table = []
    for n in (1, 2, 3, 4):
        xh = workloads.config(n)
        if xh.dtype == np.uint16:
            x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            x = torch.from_numpy(xh).cuda()
        del xh
        y = torch.empty_like(x)
        rows, cols = x.shape
        nbytes = rows * cols * x.element_size() * 2
        reps = 200 if n == 1 else 30
        entry = {"workload": n, "rows": rows, "cols": cols, "dtype": str(x.dtype).replace("torch.", ""),
                 "shape": list(ons.os_forward_plan(cols, x.dtype)), "algorithmic_bytes": nbytes}
        for name, fn in (("online", lambda: ons.os_softmax_forward(x, out=y)),
                         ("online_lse", lambda: ons.os_softmax_forward_lse(x, out=y)),
                         ("safe_3pass", lambda: ons.safe_softmax_forward(x, out=y)),
                         ("copy", lambda: ons.os_device_copy(x, y))):
            t, te = measure(fn, reps)
            entry[name] = {"us": round(t * 1e6, 2), "GBs": round(nbytes / t / 1e9, 1),
                           "pct_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1),
                           "us_eager": round(te * 1e6, 2)}
        entry["online"]["rows_per_s"] = round(rows / (entry["online"]["us"] * 1e-6), 1)
        tf = flushed(lambda: ons.os_softmax_forward(x, out=y))
        entry["online"]["us_flushed"] = round(tf * 1e6, 2)
        entry["online"]["pct_peak_flushed"] = round(100 * nbytes / tf / 1e9 / PEAK_HBM_GBS, 1)
        table.append(entry)
        del x, y
    xt = torch.from_numpy(workloads.config(5)).cuda()
    rows, cols = xt.shape
    t, te = measure(lambda: ons.os_softmax_topk(xt, workloads.TOPK_K), 200)
    nbytes = rows * cols * 4 + rows * workloads.TOPK_K * 8
    entry = {"workload": 5, "rows": rows, "cols": cols, "dtype": "float32", "K": workloads.TOPK_K,
             "algorithmic_bytes": nbytes,
             "topk": {"us": round(t * 1e6, 2), "GBs": round(nbytes / t / 1e9, 1),
                      "pct_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1),
                      "rows_per_s": round(rows / t, 1), "us_eager": round(te * 1e6, 2)}}
    tf = flushed(lambda: ons.os_softmax_topk(xt, workloads.TOPK_K))
    entry["topk"]["us_flushed"] = round(tf * 1e6, 2)
    entry["topk"]["pct_peak_flushed"] = round(100 * nbytes / tf / 1e9 / PEAK_HBM_GBS, 1)
    # the same logits rounded to bf16 (half the bytes to read)
    xb = xt.to(torch.bfloat16)
    nb16 = rows * cols * 2 + rows * workloads.TOPK_K * 8
    tb, _ = measure(lambda: ons.os_softmax_topk(xb, workloads.TOPK_K), 200)
    tbf = flushed(lambda: ons.os_softmax_topk(xb, workloads.TOPK_K))
    entry["topk_bf16"] = {"us": round(tb * 1e6, 2), "GBs": round(nb16 / tb / 1e9, 1),
                          "pct_peak": round(100 * nb16 / tb / 1e9 / PEAK_HBM_GBS, 1),
                          "us_flushed": round(tbf * 1e6, 2), "algorithmic_bytes": nb16}
    del xb
    # the unfused pipelines of the fusion comparison: softmax written out, then
    # top-K selection over the probabilities (online: 2R+1W then 1R; safe:
    # 3R+1W then 1R; naive: 2R+1W then 1R)
    yt = torch.empty_like(xt)
    for name, fwd in (("unfused_online", ons.os_softmax_forward), ("unfused_safe", ons.safe_softmax_forward),
                      ("unfused_naive", ons.naive_softmax_forward)):
        def pipeline(fwd=fwd):
            fwd(xt, out=yt)
            ons.os_topk_select(yt, workloads.TOPK_K)
        tu, tue = measure(pipeline, 100)
        tuf = flushed(pipeline)
        entry[name] = {"us": round(tu * 1e6, 2), "fused_speedup": round(tu / t, 2), "us_eager": round(tue * 1e6, 2),
                       "us_flushed": round(tuf * 1e6, 2), "fused_speedup_flushed": round(tuf / tf, 2)}
    table.append(entry)
    del xt, yt

    # few long rows: one workgroup per row against the planned split (not one
    # of the five workloads; it shows what the split-row forward is for)
    for rows, cols in ((16, 1 << 20), (1, 1 << 24)):
        x = torch.randn(rows, cols, device="cuda", generator=torch.Generator("cuda").manual_seed(rows)) * 3
        y = torch.empty_like(x)
        nbytes = rows * cols * 8
        S = ons.os_forward_split_plan(rows, cols, x.dtype)
        ws = torch.empty(ons.os_softmax_forward_workspace_bytes(rows, S), dtype=torch.uint8, device="cuda")
        tu, _ = measure(lambda: ons.os_softmax_forward(x, out=y), 10)
        ts, _ = measure(lambda: ons.os_softmax_forward_split(x, splits=S, out=y, workspace=ws), 30)
        tsf = flushed(lambda: ons.os_softmax_forward_split(x, splits=S, out=y, workspace=ws))
        table.append({"case": "split_forward", "rows": rows, "cols": cols, "dtype": "float32", "splits": S,
                      "algorithmic_bytes": nbytes,
                      "unsplit": {"us": round(tu * 1e6, 2), "pct_peak": round(100 * nbytes / tu / 1e9 / PEAK_HBM_GBS, 1)},
                      "split": {"us": round(ts * 1e6, 2), "pct_peak": round(100 * nbytes / ts / 1e9 / PEAK_HBM_GBS, 1),
                                "us_flushed": round(tsf * 1e6, 2)},
                      "speedup": round(tu / ts, 2)})
        del x, y, ws

    # rows that are not 16-byte aligned (odd lengths such as a 50257-entry
    # vocabulary): not one of the five workloads; the same kernels move them
    # as the 16-byte blocks they overlap
    for rows, cols, dt in ((4096, 32001, torch.float32), (4096, 50257, torch.float32),
                           (524288, 2047, torch.bfloat16)):
        g = torch.Generator("cuda").manual_seed(cols)
        x = (torch.randn(rows, cols, device="cuda", generator=g) * 2).to(dt)
        y = torch.empty_like(x)
        nbytes = rows * cols * x.element_size() * 2
        t, _ = measure(lambda: ons.os_softmax_forward(x, out=y), 30)
        table.append({"case": "unaligned_forward", "rows": rows, "cols": cols,
                      "dtype": str(dt).replace("torch.", ""), "algorithmic_bytes": nbytes,
                      "online": {"us": round(t * 1e6, 2), "pct_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1)}})
        del x, y
    rows, cols = 256, 50257
    x = torch.randn(rows, cols, device="cuda", generator=torch.Generator("cuda").manual_seed(cols)) * 3
    nbytes = rows * cols * 4 + rows * workloads.TOPK_K * 8
    t, _ = measure(lambda: ons.os_softmax_topk(x, workloads.TOPK_K), 200)
    table.append({"case": "unaligned_topk", "rows": rows, "cols": cols, "dtype": "float32", "K": workloads.TOPK_K,
                  "algorithmic_bytes": nbytes,
                  "topk": {"us": round(t * 1e6, 2), "pct_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1)}})
    del x

    # a mixture-of-experts router's shape (many tokens, a few hundred experts):
    # not one of the five workloads; served by the short-row top-K kernel
    for rows, cols, dt, K in ((65536, 256, torch.float32, 8), (16384, 128, torch.bfloat16, 8),
                              (65536, 64, torch.float32, 2)):
        g = torch.Generator("cuda").manual_seed(rows + cols)
        x = (torch.randn(rows, cols, device="cuda", generator=g) * 3).to(dt)
        nbytes = rows * cols * x.element_size() + rows * K * 8
        t, _ = measure(lambda: ons.os_softmax_topk_ex(x, K, 1, None), 200)
        table.append({"case": "router_topk", "rows": rows, "cols": cols, "dtype": str(dt).replace("torch.", ""),
                      "K": K, "algorithmic_bytes": nbytes,
                      "topk": {"us": round(t * 1e6, 2), "pct_peak": round(100 * nbytes / t / 1e9 / PEAK_HBM_GBS, 1)}})
        del x
    return table


if __name__ == "__main__":
    sys.exit(main())
