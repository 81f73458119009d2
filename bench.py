#!/usr/bin/env python3
"""Benchmark of the k-d tree build on one MI355X.

One step = one complete build (every round's radix passes or pivot
selections, and the subtree stage with its level-order output) of the
workload, by default the headline one:
N = 16,777,216 points, k = 3, float32, from a 64-component Gaussian mixture
with 5% of coordinates snapped to a 2^-10 grid (seed 3). --workload picks one
of the others (uniform_1m_k3, normal_4m_k16, uniform_100m_k3). Inputs, outputs
and the workspace are resident in HBM before the timed region starts.

Prints ONE JSON line on stdout (progress goes to stderr):
  value      whole-job build throughput, Mpoints/s (= N / seconds per build)
  roofline   HBM roofline of the dominant kernel (the kind with the largest
             time per build): its algorithmic bytes per launch (every array it
             must read or write, once, as the library counts them) / its
             average launch duration (HIP events on the build's stream),
             against the 8 TB/s peak; `traffic` is its measured HBM bytes per
             launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, each scaled by the
             same counter on a plain 256 MiB copy). Flat extra fields give the
             same figures for the whole build (build_*) and for the global sort
             and tag-update passes together (passes_*), and the dominant
             kernel's VALU issue rate (valu_issue_frac, a diagnostic)
  kernels    per kernel kind: launches, time, algorithmic bytes and GB/s, and
             the counter-measured bytes and GB/s beside them
  cpu_baseline  the CPU oracle on bounded samples of the same recipe: all
             host threads (value) and one thread, with the CPU model
  graph      the same build captured once into a HIP graph and replayed
             --steps times (ms_per_step and Mpoints/s); value above stays the
             eager one (--no-graph skips it)

With --widest it times the split-widest-dimension build of the same workload
instead (value, roofline and cpu_baseline as above, for that variant).

With --unique it times the duplicate-removal pre-pass on the same workload
(kept indices of the distinct tuples), the numpy oracle as cpu_baseline.

With --knn it instead times the K-nearest-neighbour query over the headline
tree (the tree is built once, untimed): --knn-queries query points drawn with
the workload's recipe, K = --knn-k; value in Mqueries/s, the roofline from the
bytes of the tree points each search examined, and the brute-force oracle on a
few sampled queries as cpu_baseline.
"""
import argparse
import csv
import glob
import json
import os
import re
import shutil
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published figure
# 32-bit VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, in T lane-ops/s
VALU_PEAK_TLANE = 256 * 4 * 16 * 2.4e9 / 1e12
COPY_BYTES = 256 << 20  # the --calibration-copy dispatch reads and writes this much
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, sample_all, sample_one, widest=False):
    """The oracle (never tuned for speed) on two bounded samples of the
    workload's recipe and seed: all host threads on sample_all points (the
    reported value), then one thread on sample_one points."""
    import oracle  # test infrastructure, used only for this reported baseline
    from tree_construction_amd import datagen
    w = datagen.WORKLOADS[name]
    lib = oracle.load_lib()
    threads = oracle.max_threads(lib)  # before any run pins the count

    def timed(n, nthreads):
        pts = datagen.cached(name) if n == w.n else datagen.generate(name, n=n)
        t0 = time.perf_counter()
        if widest:
            oracle.build_tree_widest(pts, nthreads=nthreads)
        else:
            oracle.build_tree(pts, nthreads=nthreads)
        return time.perf_counter() - t0

    n_all, n_one = min(sample_all, w.n), min(sample_one, w.n)
    dt_all = timed(n_all, threads)
    dt_one = timed(n_one, 1)
    return {"value": round(n_all / dt_all / 1e6, 3), "unit": "Mpoints/s", "cores": threads, "kind": "oracle",
            "sample": "%s recipe and seed at N=%d (k=%d), %d threads, %.1f s wall; single thread at N=%d, %.1f s"
                      % (name, n_all, w.k, threads, dt_all, n_one, dt_one),
            "single_thread_value": round(n_one / dt_one / 1e6, 3),
            "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def knn_cpu_baseline(pts, qs, K, sample):
    from oracle import knn as knn_oracle  # test infrastructure, used only for this baseline
    t0 = time.perf_counter()
    knn_oracle.knn(pts, qs[:sample], K)
    dt = time.perf_counter() - t0
    return {"value": round(sample / dt / 1e6, 9), "unit": "Mqueries/s", "cores": 1, "kind": "oracle",
            "sample": "brute force (numpy, float32) for the first %d queries against all %d points, "
                      "%.1f s wall" % (sample, len(pts), dt)}


def run_knn(args):
    import torch
    from tree_construction_amd import datagen, kdt
    name = args.workload or datagen.HEADLINE
    pts = datagen.cached(name)
    qs = datagen.generate(name, n=args.knn_queries)  # same recipe and seed, other draws
    dev = torch.device("cuda:0")
    x = torch.from_numpy(pts).to(dev)
    q = torch.from_numpy(qs).to(dev)
    n, k = pts.shape
    Q, K = len(qs), args.knn_k
    log("bench: building the %s tree (untimed)%s" % (name, ", split widest dimension" if args.widest else ""))
    dims = None
    if args.widest:
        perm, tree, dims = kdt.build_widest(x)
    else:
        perm, tree = kdt.build(x)
    idx = torch.empty((Q, K), dtype=torch.int32, device=dev)
    d2 = torch.empty((Q, K), dtype=torch.float32, device=dev)
    visits = torch.empty(Q, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    kdt.knn(tree, perm, q, K, idx, d2, visits, dims=dims)
    torch.cuda.synchronize(dev)
    v = visits.cpu().numpy()
    examined = float(v.astype(np.float64).sum())
    for _ in range(args.warmup):
        kdt.knn(tree, perm, q, K, idx, d2, dims=dims)

    def timed(qq):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        start.record(stream)
        for _ in range(args.steps):
            kdt.knn(tree, perm, qq, K, dims=dims)
        stop.record(stream)
        torch.cuda.synchronize(dev)
        return start.elapsed_time(stop) / args.steps

    log("bench: timing %d kNN passes (Q=%d, K=%d)" % (args.steps, Q, K))
    ms = timed(q)
    # the spread of the work: the pass without its 100 most expensive
    # queries, and the most expensive one alone
    order = np.argsort(-v, kind="stable")
    rest_ms = timed(q[torch.from_numpy(np.sort(order[100:])).to(dev)].contiguous())
    worst_ms = timed(q[int(order[0]):int(order[0]) + 1].contiguous())
    spread = {"mean": round(examined / Q, 2), "p50": int(np.percentile(v, 50)),
              "p99": int(np.percentile(v, 99)), "max": int(v.max()),
              "ms_without_100_most_expensive": round(rest_ms, 4),
              "ms_most_expensive_alone": round(worst_ms, 4)}
    log("bench: examined points per query %s" % spread)
    # algorithmic bytes of one pass: every examined tree point's coordinates,
    # the queries, and the two outputs
    nbytes = examined * 4 * k + Q * (4.0 * k + 8.0 * K)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("bench: %.3f ms per pass, %.1f Mqueries/s, %.1f points examined per query, %.1f GB/s"
        % (ms, Q / ms / 1e3, examined / Q, gbs))
    base = None if args.no_cpu_baseline else knn_cpu_baseline(pts, qs, K, args.knn_cpu_sample)
    if base:
        log("  %s" % base)
    out = {
        "metric": "k-d tree kNN queries (K=%d) per second over the N=16M k=3 %stree" % (
            K, "split-widest " if args.widest else ""),
        "value": round(Q / ms / 1e3, 3),
        "unit": "Mqueries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "knn over %s%s" % (name, " (split-widest tree)" if args.widest else ""),
                   "n_points": n, "k": k, "queries": Q, "K": K,
                   "queries_from": "the workload's recipe and seed, %d further draws" % Q},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "k_knn",
                     "points_examined_per_query": spread,
                     "bytes_per_launch": int(nbytes)},
        "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


def run_unique(args):
    import torch
    from tree_construction_amd import datagen, kdt
    name = args.workload or datagen.HEADLINE
    w = datagen.WORKLOADS[name]
    pts = datagen.cached(name)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(pts).to(dev)
    n, k = pts.shape
    finder = kdt.UniqueFinder(n, k, dev)
    keep = torch.empty(n, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        finder.run(x, keep)
    torch.cuda.synchronize(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        finder.run(x, keep)
    stop.record(stream)
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(stop) / args.steps
    distinct = int(finder.count.item())
    log("bench: %.3f ms per pass, %.1f Mpoints/s, %d distinct of %d" % (ms, n / ms / 1e3, distinct, n))
    agg = {}
    for _ in range(args.steps):
        for kind, rec in finder.run_profiled(x, keep).items():
            a = agg.setdefault(kind, {"launches": 0, "ms": 0.0, "bytes": 0.0})
            for f in a:
                a[f] += rec[f]
    kernels = {kk: {"launches_per_pass": a["launches"] // args.steps, "avg_us": round(a["ms"] / a["launches"] * 1e3, 2),
                    "ms_per_pass": round(a["ms"] / args.steps, 4),
                    "GBps": round(a["bytes"] / (a["ms"] * 1e-3) / 1e9, 1) if a["ms"] > 0 else 0.0}
               for kk, a in agg.items() if a["launches"]}
    for kk, kv in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_pass"]):
        log("  %-36s %4d/pass  avg %8.2f us  %8.1f GB/s  %.3f ms/pass"
            % (kk, kv["launches_per_pass"], kv["avg_us"], kv["GBps"], kv["ms_per_pass"]))
    dom = max(kernels, key=lambda kk: kernels[kk]["ms_per_pass"])
    base = None
    if not args.no_cpu_baseline:
        from oracle import unique as unique_oracle  # test infrastructure, used only for this baseline
        t0 = time.perf_counter()
        unique_oracle.unique_indices(pts)
        dt = time.perf_counter() - t0
        base = {"value": round(n / dt / 1e6, 3), "unit": "Mpoints/s", "cores": 1, "kind": "oracle",
                "sample": "the whole workload %s (numpy), %.1f s wall" % (name, dt)}
        log("  %s" % base)
    out = {
        "metric": "duplicate removal Mpoints/s at N=16M k=3 fp32",
        "value": round(n / ms / 1e3, 2), "unit": "Mpoints/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "unique over %s" % name, "n_points": n, "k": k, "distinct": distinct,
                   "description": w.note},
        "roofline": {"bound": "hbm", "achieved": kernels[dom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernels[dom]["GBps"] / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
                     "avg_us": kernels[dom]["avg_us"]},
        "cpu_baseline": base,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def kernel_short_name(name):
    """'void (anonymous namespace)::k_x<1, 2>((anonymous namespace)::Args)' -> 'k_x<1, 2>'."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name).strip()


PMC_RUNS = (("FETCH_SIZE", "SQ_INSTS_VALU"), ("WRITE_SIZE",))  # within one run's counter limits


def counter_runs(workload, widest=False):
    """Per kernel kind, the summed counters of two rocprofv3 --pmc runs of this
    benchmark (FETCH_SIZE with SQ_INSTS_VALU, then WRITE_SIZE) over its
    builds, each HBM counter scaled by what it reads for a plain 256 MiB copy
    (KiB -> bytes). Returns ({kind: {"fetch", "write", "valu", "dispatches"}},
    {counter: scale}, builds) or None if rocprofv3 is unavailable or fails."""
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None
    builds = 2  # --warmup 1 --steps 1 below
    kinds, scales = {}, {}
    field = {"FETCH_SIZE": "fetch", "WRITE_SIZE": "write", "SQ_INSTS_VALU": "valu"}
    with tempfile.TemporaryDirectory(prefix="kdt_pmc_") as tmp:
        for counters in PMC_RUNS:
            d = os.path.join(tmp, counters[0])
            cmd = ["timeout", "-s", "KILL", "300", prof, "--pmc", *counters, "--output-format", "csv",
                   "-d", d, "-o", "kdt", "--", sys.executable, os.path.abspath(__file__),
                   "--workload", workload, "--steps", "1", "--warmup", "1", "--no-profile", "--no-graph",
                   "--no-cpu-baseline", "--no-counters", "--calibration-copy"] + (["--widest"] if widest else [])
            r = subprocess.run(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)
            files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
            if r.returncode != 0 or not files:
                log("bench: %s counter run failed (rc %d)" % ("+".join(counters), r.returncode))
                return None
            copy = {}
            with open(files[0]) as f:
                for row in csv.DictReader(f):
                    cname = row.get("Counter_Name")
                    if cname not in counters:
                        continue
                    kname = kernel_short_name(row["Kernel_Name"])
                    val = float(row["Counter_Value"])
                    if kname == COPY_KERNEL:
                        copy.setdefault(cname, val)
                        continue
                    rec = kinds.setdefault(kname, {"fetch": 0.0, "write": 0.0, "valu": 0.0, "dispatches": 0})
                    rec[field[cname]] += val
                    if cname == "FETCH_SIZE":  # one row per dispatch and counter
                        rec["dispatches"] += 1
            for cname in counters:
                if cname in ("FETCH_SIZE", "WRITE_SIZE"):
                    if cname not in copy or copy[cname] <= 0:
                        log("bench: no %s reading for the calibration copy" % cname)
                        return None
                    scales[cname] = (COPY_BYTES / 1024.0) / copy[cname]
    for rec in kinds.values():
        rec["fetch"] *= 1024.0 * scales["FETCH_SIZE"]
        rec["write"] *= 1024.0 * scales["WRITE_SIZE"]
    return kinds, scales, builds


# Kernel kinds of the global phase: presort, per-round re-sorts and selects,
# their scans, the pivots and the split-widest domain kernels (everything but
# the subtree stage and the single-point case).
GLOBAL_PASS_PREFIXES = ("k_sort_", "k_part_", "k_pivots", "k_chunk_scan", "k_first_digits", "k_planar_records", "k_widest_level",
                        "k_box_", "k_zero")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1 << 22,
                    help="points of the all-threads CPU oracle run (the same recipe and seed)")
    ap.add_argument("--cpu-sample-one", type=int, default=1 << 20,
                    help="points of the single-thread CPU oracle run")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event loop")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the build captured into a HIP graph and replayed")
    ap.add_argument("--no-counters", action="store_true",
                    help="skip the rocprofv3 counter runs behind roofline.traffic and the kernels' counter bytes")
    ap.add_argument("--widest", action="store_true", help="time the split-widest-dimension build")
    ap.add_argument("--unique", action="store_true", help="time the duplicate-removal pre-pass")
    ap.add_argument("--knn", action="store_true", help="time the kNN query instead of the build")
    ap.add_argument("--knn-queries", type=int, default=1 << 20)
    ap.add_argument("--knn-k", type=int, default=8)
    ap.add_argument("--knn-cpu-sample", type=int, default=8, help="queries the brute-force baseline runs")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy, the reference "
                         "dispatch for scaling hardware traffic counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py: the k-d tree path runs on one GPU only (no multi-GPU path); "
            "run it with --gpus 1")
        sys.exit(2)
    if args.knn:
        run_knn(args)
        return
    if args.unique:
        run_unique(args)
        return

    import torch
    from tree_construction_amd import datagen, kdt

    name = args.workload or datagen.HEADLINE
    w = datagen.WORKLOADS[name]
    log("bench: generating %s (%s)" % (name, w.note))
    pts = datagen.cached(name)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(pts).to(dev)
    n, k = pts.shape
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    tree = torch.empty_like(x)
    if args.widest:
        wb = kdt.WidestBuilder(n, k, dev)
        dims = torch.empty(n, dtype=torch.int32, device=dev)

        class _Widest:  # the same two calls as kdt.Builder
            @staticmethod
            def build(x_, perm_, tree_):
                return wb.build(x_, perm_, tree_, dims)

            @staticmethod
            def build_profiled(x_, perm_, tree_):
                return wb.build_profiled(x_, perm_, tree_, dims)
        builder = _Widest()
    else:
        builder = kdt.Builder(n, k, dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize(dev)

    if args.calibration_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize(dev)
        del src, dst

    log("bench: %d warmup builds" % args.warmup)
    for _ in range(args.warmup):
        builder.build(x, perm, tree)
    torch.cuda.synchronize(dev)

    log("bench: timing %d builds" % args.steps)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        builder.build(x, perm, tree)
    stop.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps
    value = n / (ms_per_step * 1e-3) / 1e6
    log("bench: %.3f ms/build (wall %.3f ms), %.1f Mpoints/s"
        % (ms_per_step, wall * 1e3 / args.steps, value))

    graph = None
    if not args.no_graph:
        # The same build captured once into a HIP graph and replayed: the
        # kernels are the same, the host's per-launch work is gone (what a
        # caller that rebuilds in fixed buffers pays).
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            builder.build(x, perm, tree)
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            builder.build(x, perm, tree)
        g.replay()
        torch.cuda.synchronize(dev)
        start.record(stream)
        for _ in range(args.steps):
            g.replay()
        stop.record(stream)
        torch.cuda.synchronize(dev)
        gms = start.elapsed_time(stop) / args.steps
        graph = {"ms_per_step": round(gms, 4), "value": round(n / (gms * 1e-3) / 1e6, 2), "unit": "Mpoints/s",
                 "note": "one build captured into a HIP graph, %d replays" % args.steps}
        log("bench: graph replay %.3f ms/build, %.1f Mpoints/s" % (gms, graph["value"]))
        del g

    roofline, kernels = None, None
    if not args.no_profile:
        log("bench: per-kernel event timing over %d builds" % args.steps)
        agg = {}
        for _ in range(args.steps):
            for kind, rec in builder.build_profiled(x, perm, tree).items():
                a = agg.setdefault(kind, {"launches": 0, "ms": 0.0, "bytes": 0.0})
                for f in a:
                    a[f] += rec[f]
        kernels = {}
        for kind, a in agg.items():
            if a["launches"] == 0:
                continue
            per_launch_ms = a["ms"] / a["launches"]
            gbs = a["bytes"] / (a["ms"] * 1e-3) / 1e9 if a["ms"] > 0 else 0.0
            kernels[kind] = {"launches_per_build": a["launches"] // args.steps,
                             "avg_us": round(per_launch_ms * 1e3, 2),
                             "ms_per_build": round(a["ms"] / args.steps, 4),
                             "bytes_per_launch": int(a["bytes"] / a["launches"]),
                             "bytes_per_build": int(a["bytes"] / args.steps),
                             "GBps": round(gbs, 1)}
        dom = max(kernels, key=lambda kk: kernels[kk]["ms_per_build"])
        d = kernels[dom]
        achieved = d["GBps"]
        # HBM roofline of the dominant kernel from its algorithmic bytes
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": dom, "avg_us": d["avg_us"], "bytes_per_launch": d["bytes_per_launch"]}
        # the whole build: every kernel's algorithmic bytes over the build time
        build_bytes = sum(kv["bytes_per_build"] for kv in kernels.values())
        build_gbs = build_bytes / (ms_per_step * 1e-3) / 1e9
        roofline.update({"build_bytes": build_bytes, "build_GBps": round(build_gbs, 1),
                         "build_frac": round(build_gbs / HBM_PEAK_GBS, 4)})
        # the global sort and tag-update passes together (the subtree stage,
        # which finishes the last rounds in LDS, is not among them)
        passes = [kk for kk in kernels if kk.startswith(GLOBAL_PASS_PREFIXES)]
        pass_bytes = sum(kernels[kk]["bytes_per_build"] for kk in passes)
        pass_ms = sum(kernels[kk]["ms_per_build"] for kk in passes)
        if pass_ms > 0:
            roofline.update({"passes_ms_per_build": round(pass_ms, 4),
                             "passes_GBps": round(pass_bytes / (pass_ms * 1e-3) / 1e9, 1),
                             "passes_frac": round(pass_bytes / (pass_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        for kind, kv in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_build"]):
            log("  %-36s %4d/build  avg %8.2f us  %8.1f GB/s  %.3f ms/build"
                % (kind, kv["launches_per_build"], kv["avg_us"], kv["GBps"], kv["ms_per_build"]))
        log("  whole build: %.2f GB algorithmic, %.1f GB/s (%.1f%% of peak)"
            % (build_bytes / 1e9, build_gbs, 100 * build_gbs / HBM_PEAK_GBS))
        if not args.no_counters:
            log("bench: rocprofv3 counter runs (FETCH_SIZE + SQ_INSTS_VALU, then WRITE_SIZE)")
            got = counter_runs(name, widest=args.widest)
            if got:
                ckinds, scales, builds = got
                roofline["counter_scale_fetch"] = round(scales["FETCH_SIZE"], 3)
                roofline["counter_scale_write"] = round(scales["WRITE_SIZE"], 3)
                counter_build, counter_pass = 0.0, 0.0
                for kind, kv in kernels.items():
                    c = ckinds.get(kind)
                    if not c:
                        continue
                    cb = (c["fetch"] + c["write"]) / builds  # per build
                    counter_build += cb
                    if kind in passes:
                        counter_pass += cb
                    kv.update({"counter_fetch_per_build": int(c["fetch"] / builds),
                               "counter_write_per_build": int(c["write"] / builds),
                               "counter_GBps": round(cb / (kv["ms_per_build"] * 1e-3) / 1e9, 1),
                               "counter_over_algorithmic": round(cb / kv["bytes_per_build"], 3)
                               if kv["bytes_per_build"] else None,
                               "valu_per_launch": int(c["valu"] / max(c["dispatches"], 1))})
                    log("  %-36s counters %8.1f MB/build (%.2fx algorithmic), %8.1f GB/s"
                        % (kind, cb / 1e6, kv["counter_over_algorithmic"] or 0.0, kv["counter_GBps"]))
                c = ckinds.get(dom)
                if c and c["dispatches"]:
                    per_launch = (c["fetch"] + c["write"]) / c["dispatches"]
                    inst = c["valu"] / c["dispatches"]
                    lane_ops = inst * 64 / (d["avg_us"] * 1e-6) / 1e12
                    roofline.update({"traffic": int(per_launch),
                                     "traffic_fetch": int(c["fetch"] / c["dispatches"]),
                                     "traffic_write": int(c["write"] / c["dispatches"]),
                                     "traffic_over_algorithmic": round(per_launch / d["bytes_per_launch"], 3),
                                     "valu_instructions_per_launch": int(inst),
                                     "valu_issue_frac": round(lane_ops / VALU_PEAK_TLANE, 4)})
                roofline.update({"counter_build_bytes": int(counter_build),
                                 "counter_build_GBps": round(counter_build / (ms_per_step * 1e-3) / 1e9, 1)})
                if pass_ms > 0:
                    roofline["passes_counter_GBps"] = round(counter_pass / (pass_ms * 1e-3) / 1e9, 1)
                log("  dominant %s: traffic %s B/launch (%.2fx algorithmic); whole build %.2f GB counted"
                    % (dom, roofline["traffic"], roofline.get("traffic_over_algorithmic") or 0.0,
                       counter_build / 1e9))

    base = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline (all threads on %d points, one thread on %d)"
            % (min(args.cpu_sample, n), min(args.cpu_sample_one, n)))
        base = cpu_baseline(name, args.cpu_sample, args.cpu_sample_one, widest=args.widest)
        log("  %s" % base)

    if name == datagen.HEADLINE:
        metric = ("k-d tree (split widest dimension) build Mpoints/s at N=16M k=3 fp32; achieved HBM GB/s vs peak"
                  if args.widest else "k-d tree build Mpoints/s at N=16M k=3 fp32; achieved HBM GB/s vs peak")
    else:
        metric = "k-d tree %sbuild Mpoints/s at N=%d k=%d fp32 (%s); achieved HBM GB/s vs peak" % (
            "(split widest dimension) " if args.widest else "", n, k, name)
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "Mpoints/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "n_points": n, "k": k, "coords": "f32",
                   "description": w.note},
        "roofline": roofline,
        "cpu_baseline": base,
        "graph": graph,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
