#!/usr/bin/env python3
"""Throughput of the MSDA forward core on one MI355X.

One step = one msda_forward call over one batch of the Deformable-DETR
encoder workload (N=2, 4 levels (100,167),(50,84),(25,42),(13,21), S=Lq=22223,
M=8, D=32, L=4, P=4, fp32), inputs already resident in HBM.  With
``--op backward`` a step is one msda_backward call instead (grad_value fill
plus the gradient kernel) on the same inputs and an N(0,1) output gradient;
with ``--op forward_fused`` one msda_forward_fused call on the same draws
before the front end (reference points, offsets, logits), and the unfused
pipeline (torch softmax + add, then msda_forward) is timed beside it; with
``--op forward_pruned`` one msda_forward_pruned call at ``--prune-threshold``
(the fraction of samples it drops and the unpruned kernel's time on the same
inputs are reported beside it).
Queries are visited in a Z-order (Morton) order of the pixels when the
workload's queries are the pyramid's pixel centres, except in the 2D pruned
forward (``--query-order``; the order depends only on the level shapes, so it
is built once, before the timed steps, like any per-shape plan: ``value`` and
the kernel time exclude its build, whose own GPU time is reported as
``query_order_build_us``, and ``value_with_query_order_build_every_step`` is
the rate if it were rebuilt at every step); every output is the same as in
the raw query order, which ``--query-order none`` times.
Steps cycle over several distinct copies of the inputs whose total exceeds
twice the 256 MB Infinity Cache, so each step reads its inputs from HBM
rather than from a cache warmed by the previous step.

Prints one JSON line: sampled points/s over the timed steps (wall clock,
synchronised on both sides), achieved effective HBM GB/s of the kernel against
the 8 TB/s peak (roofline; the kernel time is the mean of the same number of
launches run back to back behind a GPU spin and bracketed by one pair of HIP
events on the launch stream; ``kernel_us_single`` gives min, median, p90 and
max of launches timed one at a time), the gathered bytes/s against the measured
ceiling of the same access pattern (roofline.gather, from the calibration
kernels of include/msda_calib.h), the oracle's CPU throughput on the same
inputs over the host's threads and on one core (cpu_baseline), and the
counter traffic recorded for this kernel under profiles/ when it is still
current.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sampled points/sec + achieved HBM GB/s (DETR encoder shape, 1 MI355X)"
METRIC_BACKWARD = ("backward sampled points/sec + achieved HBM GB/s "
                   "(DETR encoder shape, 1 MI355X)")
METRIC_PRUNED = ("pruned forward sampled points/sec + achieved HBM GB/s "
                 "(DETR encoder shape, 1 MI355X)")
METRIC_FUSED = ("fused front end + forward sampled points/sec + achieved HBM GB/s "
                "(DETR encoder shape, 1 MI355X)")
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "scale_deformable_attention_02_amd", "csrc")
COUNTERS_FILES = {
    "forward": os.path.join(ROOT, "profiles", "msda_forward_counters.json"),
    "forward_fused": os.path.join(ROOT, "profiles", "msda_forward_fused_counters.json"),
    "forward_pruned": os.path.join(ROOT, "profiles", "msda_forward_pruned_counters.json"),
    "backward": os.path.join(ROOT, "profiles", "msda_backward_counters.json"),
    "linear": os.path.join(ROOT, "profiles", "msda_linear_counters.json"),
}
KERNEL_SOURCES = {
    "forward": [os.path.join(CSRC, "msda_device.hpp"), os.path.join(CSRC, "msda_forward_impl.hpp"),
                os.path.join(CSRC, "msda_api.hip")],
    "forward_fused": [os.path.join(CSRC, "msda_device.hpp"),
                      os.path.join(CSRC, "msda_forward_impl.hpp"),
                      os.path.join(CSRC, "msda_api_fused.hip")],
    "forward_pruned": [os.path.join(CSRC, "msda_device.hpp"),
                       os.path.join(CSRC, "msda_forward_impl.hpp"),
                       os.path.join(CSRC, "msda_api_pruned.hip")],
    "backward": [os.path.join(CSRC, "msda_device.hpp"), os.path.join(CSRC, "msda_backward.hpp"),
                 os.path.join(CSRC, "msda_backward_api.hip")],
    "linear": [os.path.join(CSRC, "msda_device.hpp"), os.path.join(CSRC, "msda_linear.hip")],
}


def kernel_source_digest(op: str = "forward") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[op]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def byte_counts(w):
    """Algorithmic bytes of one launch.

    U (compulsory): locations + weights + out + value, each moved once (value
    capped at the gathered bytes when few queries touch it).
    G (gathered): every corner row read once per sample, plus the streams.
    """
    samples = w.sampled_points
    corners = 4 if w.dims == 2 else 8
    loc = samples * w.dims * 4
    attw = samples * 4
    out = w.N * w.queries_per_image * w.M * w.D * w.out_itemsize
    value = w.N * w.S * w.M * w.D * w.value_itemsize
    gathered_value = samples * corners * w.D * w.value_itemsize
    U = loc + attw + out + min(value, gathered_value)
    G = loc + attw + out + gathered_value
    return U, G


def backward_byte_counts(w):
    """Algorithmic bytes of one backward call (fill + gradient kernel).

    U (compulsory): locations, weights, grad_out and value read once (value
    capped at the gathered bytes), grad_locations, grad_weights and the fp32
    grad_value written once.
    G (gathered): every corner row of value read once per sample and every
    corner row of grad_value updated once per sample (read-modify-write in
    the L2 atomics: 2x its fp32 bytes), plus the streams.
    """
    samples = w.sampled_points
    corners = 4 if w.dims == 2 else 8
    loc = samples * w.dims * 4
    attw = samples * 4
    gout = w.N * w.queries_per_image * w.M * w.D * w.value_itemsize
    value = w.N * w.S * w.M * w.D * w.value_itemsize
    gvalue = w.N * w.S * w.M * w.D * 4
    gathered_value = samples * corners * w.D * w.value_itemsize
    scatter = samples * corners * w.D * 4
    streams = 2 * (loc + attw) + gout
    U = streams + min(value, gathered_value) + min(gvalue, scatter)
    G = streams + gathered_value + 2 * scatter
    return U, G


def counters_for(workload_name: str, op: str = "forward", query_order: str = "none"):
    """Per-launch HBM traffic from committed rocprofv3 counters, if they were
    taken from the current kernel sources with the same query order."""
    path = COUNTERS_FILES[op]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_source_digest") != kernel_source_digest(op):
        return None
    entry = data.get("workloads", {}).get(workload_name)
    if not entry or entry.get("query_order", "none") != query_order:
        return None
    return entry.get("traffic_bytes_per_launch")


def resolve_query_order(requested: str, w, op: str):
    """The visit order a run uses: "none", "interleaved" or "levels" (the
    pixel-centre orders), "points" (the order of one point per query: the
    first image's first sampling location of each query), or None when a
    pixel-centre order is requested for queries that are not pixel centres.
    "auto" is the measured best: the interleaved Z-order for pixel-centre
    queries, except the 2D pruned forward, which runs slower with it."""
    if requested == "auto":
        best = w.queries == "pixel_centres" and not (op == "forward_pruned" and w.dims == 2)
        return "interleaved" if best else "none"
    if requested in ("levels", "interleaved") and w.queries != "pixel_centres":
        return None
    return requested


def launch_distribution(step, n, stream):
    """min / median / p90 / max (us) of ``n`` launches of ``step``, each timed
    alone: an event pair around it, then a synchronize before the next, so a
    figure includes one launch's dispatch latency and no neighbour's tail."""
    import torch

    ts = []
    for i in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    ts.sort()
    return {"n": n, "min": ts[0], "median": ts[n // 2], "p90": ts[min(n - 1, (9 * n) // 10)],
            "max": ts[-1]}


def launch_times(step, n, stream, host_us_per_step):
    """Mean duration (s) of ``n`` back-to-back launches of ``step``.

    The launches are queued behind a GPU spin (torch.cuda._sleep) that lasts
    longer than the host needs to enqueue them, so they run back to back; one
    event pair brackets all of them.  Neither the host's enqueue time (which
    exceeds a short kernel) nor per-launch event markers (a few microseconds
    each) enter the figure; the small dispatch gaps between launches do."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    try:
        # spin cycles per microsecond, measured
        a.record(stream)
        torch.cuda._sleep(1_000_000)
        b.record(stream)
        torch.cuda.synchronize()
        cyc_per_us = 1_000_000 / max(a.elapsed_time(b) * 1e3, 1.0)
        backlog_us = min(2.0 * n * host_us_per_step + 2000.0, 2e6)
        torch.cuda._sleep(int(backlog_us * cyc_per_us))
    except (AttributeError, RuntimeError):
        pass
    a.record(stream)
    for i in range(n):
        step(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / n


# Windows of the random-row calibration: L1-, L2- and Infinity-Cache-resident
# and HBM-scale (powers of two).
CALIB_WINDOWS = {"l1": 16 << 10, "l2": 2 << 20, "mall": 32 << 20, "hbm": 1 << 30}
CALIB_LDS_MODES = {"lds_rows": 0, "lds_row_pairs": 1, "lds_broadcast": 2,
                   "lds_half_rows_same_banks": 3, "lds_half_rows_other_banks": 4,
                   "lds_corner_quads_swizzled": 5, "lds_corner_quads": 6,
                   "lds_corner_quads_odd_pitch": 7, "lds_slot_words": 8}
CLOCK_GHZ = 2.4
NUM_CUS = 256


def gather_ceilings(dev, windows=CALIB_WINDOWS, lds_modes=CALIB_LDS_MODES, stream_bytes=1 << 30,
                    reps=5):
    """Measured delivery rates of the hot path's access pattern (128-byte rows
    at random positions, 8 lanes x 16 bytes each) from each memory level, and
    of a coalesced HBM read stream: GB/s and bytes per CU-clock (at the 2.4 GHz
    peak clock), the median of ``reps`` timed launches after one warm-up."""
    import torch

    from scale_deformable_attention_02_amd.binding import (calib_gather_global,
                                                           calib_gather_global_lds,
                                                           calib_gather_lds, calib_stream)

    blocks = NUM_CUS * 8
    big = max(max(windows.values()), stream_bytes)
    buf = torch.randint(0, 255, (big,), dtype=torch.uint8, device=dev)
    sink = torch.empty(blocks * 256 * 16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(launch):
        launch()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            nbytes = launch()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / 1e3)
        t = statistics.median(times)
        return {"gbps": nbytes / t / 1e9,
                "bytes_per_cu_clk": nbytes / t / (NUM_CUS * CLOCK_GHZ * 1e9)}

    out = {}
    for name, wb in windows.items():
        iters = 1024 if name in ("mall", "hbm") else 4096
        out[name] = timed(lambda: calib_gather_global(buf, wb, blocks, iters, sink))
        out[name]["window_bytes"] = wb
        if name in ("l1", "l2"):   # the same rows read half a row per 4 lanes
            out[name + "_half_rows"] = timed(
                lambda: calib_gather_global(buf, wb, blocks, iters, sink, lanes_per_row=4))
            # the same rows into LDS by the loads' LDS mode, then read back
            out[name + "_via_lds_dma"] = timed(
                lambda: calib_gather_global_lds(buf, wb, blocks, iters, sink))
    for name, mode in lds_modes.items():
        out[name] = timed(lambda: calib_gather_lds(buf, mode, blocks, 4096, sink))
    out["hbm_stream"] = timed(lambda: calib_stream(buf, stream_bytes, blocks, sink))
    del buf, sink
    return out


def bench_calib(args):
    """--op calib: the gather ceilings alone, as one JSON line."""
    import torch

    dev = torch.device("cuda:0")
    ceil = gather_ceilings(dev)
    print(json.dumps({
        "metric": "gather ceilings: random 128-byte rows per memory level (1 MI355X)",
        "value": ceil["l1"]["gbps"], "unit": "GB/s (L1-resident random rows)",
        "n_gpus": 1, "higher_is_better": True, "vs_baseline": None, "dtype": "u8",
        "data": "synthetic", "config": {"workload": "gather calibration",
                                        "clock_ghz_assumed": CLOCK_GHZ, "cus": NUM_CUS},
        "ceilings": ceil}), flush=True)
    return 0


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's guess."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads() -> int:
    """Threads for the all-cores oracle leg: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when it is set (the GPU machine's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(w, inp, max_points=60_000_000, grad_out=None, threshold=None,
                 min_seconds=10.0, max_passes=200, threads=None):
    """Time the oracle (plain C, one sample point at a time) on the same
    inputs, bounded: at most ``max_points`` sampled points per pass, passes
    repeated until ``min_seconds`` have elapsed (or ``max_passes``).  Two legs:
    the single-threaded oracle on the whole sample, and the same function over
    ``threads`` host threads, each on its own disjoint (image, query range)
    slices of the sample.  The backward oracle when ``grad_out`` is given, the
    fused-front-end oracle when ``inp`` holds reference points, offsets and
    logits."""
    import concurrent.futures

    import numpy as np

    import oracle

    fused = "reference_points" in inp
    if fused:
        fn = (oracle.msda_oracle_forward_fused if w.dims == 2
              else oracle.msda3d_oracle_forward_fused)
    elif threshold is not None:
        fn = (oracle.msda_oracle_forward_pruned if w.dims == 2
              else oracle.msda3d_oracle_forward_pruned)
    elif grad_out is None:
        fn = oracle.msda_oracle_forward if w.dims == 2 else oracle.msda3d_oracle_forward
    else:
        fn = oracle.msda_oracle_backward if w.dims == 2 else oracle.msda3d_oracle_backward
    per_query = w.M * w.L * w.P
    if w.sampled_points <= max_points:
        nb, nq = w.N, w.queries_per_image
        sample = "the whole workload"
    else:
        nb, nq = 1, max(1, max_points // per_query)
        sample = f"queries 0..{nq - 1} of image 0"
    value = inp["value"][:nb].double().numpy()
    shapes = inp["spatial_shapes"].numpy()
    starts = inp["level_start_index"].numpy()
    if fused:
        per_q = (np.ascontiguousarray(inp["reference_points"][:nb, :nq].numpy()),
                 np.ascontiguousarray(inp["sampling_offsets"][:nb, :nq].numpy()),
                 inp["attention_logits"][:nb, :nq].double().numpy())
    else:
        per_q = (np.ascontiguousarray(inp["sampling_locations"][:nb, :nq].numpy()),
                 inp["attention_weights"][:nb, :nq].double().numpy())
    if grad_out is not None:
        per_q += (grad_out[:nb, :nq].double().numpy(),)
    tail = (threshold,) if threshold is not None else ()

    def call(n0, n1, q0, q1):
        # the same entry point on images n0..n1-1, queries q0..q1-1 (the
        # value pyramid of those images is shared, read-only)
        fn(value[n0:n1], shapes, starts,
           *(np.ascontiguousarray(a[n0:n1, q0:q1]) for a in per_q), *tail)

    def timed(run):
        passes = 0
        t0 = time.perf_counter()
        while True:
            run()
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or passes >= max_passes:
                return passes, dt

    model = cpu_model()
    passes, dt = timed(lambda: call(0, nb, 0, nq))
    points = nb * nq * per_query * passes
    single = {
        "value": points / dt, "unit": "sampled points/s", "cores": 1, "kind": "oracle",
        "sample": f"{sample}, {passes} passes: {points} sampled points in {dt:.2f} s, "
                  f"single-threaded C oracle (fp64 accumulate) on {model}",
    }
    T = threads or host_threads()
    # disjoint slices: every image cut into query ranges, about 4 per thread
    pieces = max(1, (4 * T + nb - 1) // nb)
    step = max(1, -(-nq // pieces))
    jobs = [(n, n + 1, q0, min(nq, q0 + step)) for n in range(nb) for q0 in range(0, nq, step)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=T) as pool:
        def run_all():
            list(pool.map(lambda j: call(*j), jobs))
        passes_t, dt_t = timed(run_all)
    points_t = nb * nq * per_query * passes_t
    return {
        "value": points_t / dt_t, "unit": "sampled points/s", "cores": T, "kind": "oracle",
        "sample": f"{sample}, {passes_t} passes: {points_t} sampled points in {dt_t:.2f} s, "
                  f"the C oracle over {T} host threads, {len(jobs)} disjoint (image, query "
                  f"range) slices per pass, on {model}",
        "cpu_model": model,
        "single_core": single,
    }


def bench_linear(args):
    """The value projection W'_m of every pixel of the workload: y[N*S, M*D] =
    x[N*S, C] W^T + b with C = M*D, as one msda_linear call per step."""
    import torch

    from scale_deformable_attention_02_amd import msda_linear
    from scale_deformable_attention_02_amd.workloads import CONFIGS, make_linear_inputs

    w = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    R, K, N = w.N * w.S, w.M * w.D, w.M * w.D
    es = 2 if args.linear_dtype == "bf16" else 4
    flops = 2.0 * R * K * N
    U = (R * K + N * K + R * N) * es + N * 4
    copies = max(2, -(-(2 * MALL_BYTES + 1) // U))
    inp = make_linear_inputs(R, K, N, args.linear_dtype, seed=w.seed)
    sets = []
    for c in range(copies):
        x = inp["x"].to(dev) if c == 0 else sets[0][0].clone()
        sets.append((x, inp["weight"].to(dev), inp["bias"].to(dev),
                     torch.empty((R, N), dtype=x.dtype, device=dev)))

    def step(i):
        x, wt, b, y = sets[i % copies]
        msda_linear(x, wt, b, out=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_s = launch_times(step, args.steps, stream, host_s / args.steps * 1e6)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    peak_tflops = 2500.0 if args.linear_dtype == "bf16" else 157.3
    t_hbm, t_mfma = U / (HBM_PEAK_GBPS * 1e9), flops / (peak_tflops * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    achieved_gbps, achieved_tflops = U / kernel_s / 1e9, flops / kernel_s / 1e12
    roof = ({"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": achieved_gbps / HBM_PEAK_GBPS}
            if bound == "hbm" else
            {"bound": "mfma", "achieved": achieved_tflops, "peak": peak_tflops,
             "unit": "TFLOP/s", "frac": achieved_tflops / peak_tflops})
    roof["traffic"] = counters_for(w.name, "linear")
    result = {
        "metric": "value projection rows/sec + roofline (msda_linear, 1 MI355X)",
        "value": R / (wall / args.steps),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.linear_dtype,
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": {"workload": f"{w.name} value projection", "R": R, "K": K, "N": N,
                   "input_copies_cycled": copies, "parallelism": "single GPU", "op": "linear"},
        "kernel_us_mean": kernel_s * 1e6,
        "achieved_hbm_gbps": achieved_gbps,
        "achieved_tflops": achieved_tflops,
        "bytes_per_launch": {"compulsory": U},
        "flops_per_launch": flops,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import numpy as np

        from oracle import linear_oracle
        nr = min(R, 20000)
        t1 = time.perf_counter()
        linear_oracle(inp["x"][:nr], inp["weight"], inp["bias"])
        dt = time.perf_counter() - t1
        result["cpu_baseline"] = {
            "value": nr / dt, "unit": "rows/s", "cores": int(os.environ.get("OMP_NUM_THREADS", "0")
                                                            or os.cpu_count() or 1),
            "kind": "oracle",
            "sample": f"rows 0..{nr - 1}: fp64 numpy matmul ({np.__version__}) in {dt:.3f} s"}
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="detr_encoder",
                    help="workload name (default: the DETR encoder configuration)")
    ap.add_argument("--op", choices=("forward", "forward_fused", "forward_pruned", "backward",
                                     "linear", "calib"),
                    default="forward",
                    help="time the forward (default), the forward with the fused front "
                         "end, the pruned forward, the backward entry point, or the value "
                         "projection (msda_linear) of the workload's pixels")
    ap.add_argument("--linear-dtype", choices=("bf16", "f32"), default="bf16",
                    help="operand and output dtype of --op linear")
    ap.add_argument("--prune-threshold", type=float, default=None,
                    help="attention-weight threshold of --op forward_pruned "
                         "(default 0.8 / (L*P): about half the samples of softmaxed "
                         "N(0,1) logits)")
    ap.add_argument("--query-order", choices=("auto", "none", "levels", "interleaved", "points"),
                    default="auto",
                    help="visit order of the queries: a Z-order of the pixels with the "
                         "levels interleaved or level by level, a Z-order of one point per "
                         "query (the first image's first sampling locations), or none (the "
                         "raw order); auto = interleaved for pixel-centre workloads (except "
                         "the 2D pruned forward), else none")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the oracle (for profiler runs)")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the gather-ceiling calibration (roofline.gather)")
    ap.add_argument("--out-dtype", choices=("f32", "bf16"), default=None,
                    help="output dtype of the forward ops (default: the workload's)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); the core "
              "needs no communication between GPUs: shard by image, query or head and run "
              "one process per GPU", file=sys.stderr)
        return 2

    import torch

    if args.op == "linear":
        return bench_linear(args)
    if args.op == "calib":
        return bench_calib(args)

    from scale_deformable_attention_02_amd import (msda3d_backward, msda3d_forward,
                                                   msda3d_forward_fused, msda3d_forward_pruned,
                                                   msda_backward, msda_forward,
                                                   msda_forward_fused, msda_forward_pruned,
                                                   msda_query_order, msda_query_order_points)
    from scale_deformable_attention_02_amd.workloads import (CONFIGS, make_fused_inputs,
                                                             make_grad_out, make_inputs)

    w = CONFIGS[args.config]
    if args.out_dtype is not None and args.op != "backward":
        w = w.with_(out_dtype=args.out_dtype)
    dev = torch.device("cuda:0")
    backward = args.op == "backward"
    fused = args.op == "forward_fused"
    pruned = args.op == "forward_pruned"
    threshold = args.prune_threshold
    if pruned and threshold is None:
        threshold = 0.8 / (w.L * w.P)
    inp = make_fused_inputs(w) if fused else make_inputs(w)
    U, G = backward_byte_counts(w) if backward else byte_counts(w)
    if fused:  # plus the reference points, read once
        U += w.N * w.queries_per_image * w.dims * 4
        G += w.N * w.queries_per_image * w.dims * 4
    copies = max(2, -(-(2 * MALL_BYTES + 1) // U))
    base = {k: v.to(dev) for k, v in inp.items()}
    if backward:
        base["grad_out"] = make_grad_out(w).to(dev)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]

    order_kind = resolve_query_order(args.query_order, w, args.op)
    if order_kind is None:
        print(f"bench.py: --query-order {args.query_order} needs pixel-centre queries; "
              f"{w.name} has {w.queries!r}", file=sys.stderr)
        return 2
    order, order_build_us = None, None
    if order_kind == "points":
        # one point per query: the first image's first sampling location, or
        # its reference point for the fused front end (built
        # before the timed steps, like a per-batch plan; its GPU time reported)
        pts = (base["reference_points"][0] if fused
               else base["sampling_locations"][0, :, 0, 0, 0, :]).contiguous()
        order = msda_query_order_points(pts)
        torch.cuda.synchronize()
        order_build_us = launch_times(lambda i: msda_query_order_points(pts, out=order), 10,
                                      torch.cuda.current_stream(dev), 200.0) * 1e6
    elif order_kind != "none":
        # built once per pyramid shape, before the timed steps; its GPU time is
        # reported (mean of back-to-back rebuilds, host overhead excluded)
        order = msda_query_order(w.shapes, order_kind == "levels", device=dev)
        torch.cuda.synchronize()
        order_build_us = launch_times(
            lambda i: msda_query_order(w.shapes, order_kind == "levels", out=order), 10,
            torch.cuda.current_stream(dev), 200.0) * 1e6
    if backward:
        outs = [(torch.empty_like(d["value"], dtype=torch.float32),
                 torch.empty_like(d["sampling_locations"]),
                 torch.empty_like(d["attention_weights"])) for d in sets]
        bwd = msda_backward if w.dims == 2 else msda3d_backward

        def step(i):
            d = sets[i % copies]
            gv, gl, ga = outs[i % copies]
            bwd(d["value"], d["spatial_shapes"], d["level_start_index"],
                d["sampling_locations"], d["attention_weights"], d["grad_out"],
                grad_value=gv, grad_sampling_locations=gl, grad_attention_weights=ga,
                query_order=order)
    elif fused:
        out_dt = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
        outs = [torch.empty((w.N, w.queries_per_image, w.M * w.D), dtype=out_dt, device=dev)
                for _ in range(copies)]
        ffn = msda_forward_fused if w.dims == 2 else msda3d_forward_fused
        fwd = msda_forward if w.dims == 2 else msda3d_forward

        def step(i):
            d = sets[i % copies]
            ffn(d["value"], d["spatial_shapes"], d["level_start_index"], d["reference_points"],
                d["sampling_offsets"], d["attention_logits"], out=outs[i % copies],
                query_order=order)

        def unfused_step(i):
            d = sets[i % copies]
            N, Lq, M, L, P, dims = d["sampling_offsets"].shape
            loc = d["reference_points"].reshape(N, Lq, 1, 1, 1, dims) + d["sampling_offsets"]
            attw = torch.softmax(d["attention_logits"].reshape(N, Lq, M, L * P), dim=-1)
            fwd(d["value"], d["spatial_shapes"], d["level_start_index"], loc,
                attw.reshape(N, Lq, M, L, P), out=outs[i % copies], query_order=order)
    elif pruned:
        out_dt = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
        outs = [torch.empty((w.N, w.queries_per_image, w.M * w.D), dtype=out_dt, device=dev)
                for _ in range(copies)]
        pfn = msda_forward_pruned if w.dims == 2 else msda3d_forward_pruned
        fwd = msda_forward if w.dims == 2 else msda3d_forward

        def step(i):
            d = sets[i % copies]
            pfn(d["value"], d["spatial_shapes"], d["level_start_index"],
                d["sampling_locations"], d["attention_weights"], threshold,
                out=outs[i % copies], query_order=order)

        def unfused_step(i):  # the unpruned kernel on the same inputs
            d = sets[i % copies]
            fwd(d["value"], d["spatial_shapes"], d["level_start_index"],
                d["sampling_locations"], d["attention_weights"], out=outs[i % copies],
                query_order=order)
    else:
        out_dt = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
        outs = [torch.empty((w.N, w.queries_per_image, w.M * w.D), dtype=out_dt, device=dev)
                for _ in range(copies)]
        fwd = msda_forward if w.dims == 2 else msda3d_forward

        def step(i):
            d = sets[i % copies]
            fwd(d["value"], d["spatial_shapes"], d["level_start_index"],
                d["sampling_locations"], d["attention_weights"], out=outs[i % copies],
                query_order=order)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_s = launch_times(step, args.steps, stream, host_s / args.steps * 1e6)

    # back-to-back on one input set: inputs stay in L2/Infinity Cache
    warm_s = launch_times(lambda i: step(0), 20, stream, host_s / args.steps * 1e6)
    # the spread: launches timed one at a time (an event pair each, idle GPU
    # between them), inputs cycled as in the timed steps
    dist = launch_distribution(step, max(args.steps, 20), stream)

    unfused_us = None
    if fused or pruned:
        # the comparison leg (fused: the front end as separate torch passes;
        # pruned: the unpruned kernel), timed the same way as the main leg
        for i in range(3):
            unfused_step(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            unfused_step(i)
        host_u = time.perf_counter() - t1
        torch.cuda.synchronize()
        unfused_us = launch_times(unfused_step, args.steps, stream, host_u / args.steps * 1e6) * 1e6

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    points = w.sampled_points
    ms_per_step = wall / args.steps * 1e3
    achieved = U / kernel_s / 1e9
    order_label = ("none" if order is None else
                   "z-order, levels interleaved" if order_kind == "interleaved"
                   else "z-order of one point per query" if order_kind == "points"
                   else "z-order, level by level")
    # committed counters were taken with the workload's own output dtype
    traffic = (counters_for(w.name, args.op, order_label)
               if w.out_dtype == CONFIGS[w.name].out_dtype else None)
    result = {
        "metric": (METRIC_BACKWARD if backward else METRIC_FUSED if fused
                   else METRIC_PRUNED if pruned else METRIC),
        "value": points / (wall / args.steps),
        "unit": "sampled points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.value_dtype == "bf16" else "f32",
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": {
            "workload": w.name, "N": w.N, "levels": [list(s) for s in w.shapes], "S": w.S,
            "Lq": w.queries_per_image, "M": w.M, "D": w.D, "L": w.L, "P": w.P,
            "value_dtype": w.value_dtype, "out_dtype": w.out_dtype,
            "op": args.op, "input_copies_cycled": copies,
            "query_order": order_label,
            "parallelism": "single GPU",
        },
        "achieved_hbm_gbps": achieved,
        "gathered_gbps": G / kernel_s / 1e9,
        "kernel_us_mean": kernel_s * 1e6,
        "kernel_us_warm": warm_s * 1e6,
        "kernel_us_single": dist,
        "query_order_build_us": order_build_us,
        # the visit order is a per-shape plan built once before the timed
        # region: it is not in value; the rate if it were rebuilt every step
        "value_includes_query_order_build": False,
        "value_with_query_order_build_every_step": (
            w.sampled_points / (wall / args.steps + order_build_us * 1e-6)
            if order_build_us is not None else None),
        "bytes_per_launch": {"compulsory": U, "gathered": G},
        "unfused_pipeline_us_per_step": unfused_us if fused else None,
        "unpruned_us_per_step": unfused_us if pruned else None,
        "prune": ({"threshold": threshold,
                   "pruned_fraction": float((inp["attention_weights"] < threshold).double().mean()),
                   "pruned_weight_mass": float(
                       torch.where(inp["attention_weights"] < threshold,
                                   inp["attention_weights"], 0).double().sum()
                       / inp["attention_weights"].double().sum())}
                  if pruned else None),
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
    }
    if not args.no_calibration:
        # the gathered bytes per second against the measured delivery rate of
        # the same access pattern: random 128-byte rows from an L1-resident
        # window (the path corner rows take through the texture units), and
        # the other ceilings beside it
        ceil = gather_ceilings(dev, windows={"l1": CALIB_WINDOWS["l1"],
                                             "l2": CALIB_WINDOWS["l2"]},
                               lds_modes={"lds_rows": 0})
        gathered = G / kernel_s / 1e9
        result["roofline"]["gather"] = {
            "gathered_gbps": gathered,
            "ceiling": ceil["l1"]["gbps"],
            "frac": gathered / ceil["l1"]["gbps"],
            "ceiling_kind": "L1-resident random 128-byte rows (8 lanes x 16 B)",
            "l2_ceiling": ceil["l2"]["gbps"],
            "lds_ceiling": ceil["lds_rows"]["gbps"],
            "hbm_stream": ceil["hbm_stream"]["gbps"],
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(
            w, inp, grad_out=make_grad_out(w) if backward else None,
            threshold=threshold if pruned else None)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
