#!/usr/bin/env python3
"""Benchmark of the k-d tree build on one MI355X.

One step = one complete build (every round's radix passes or pivot
selections, and the subtree stage with its level-order output) of the
headline workload:
N = 16,777,216 points, k = 3, float32, from a 64-component Gaussian mixture
with 5% of coordinates snapped to a 2^-10 grid (seed 3). Inputs, outputs and
the workspace are resident in HBM before the timed region starts.

Prints ONE JSON line on stdout (progress goes to stderr):
  value      whole-job build throughput, Mpoints/s (= N / seconds per build)
  roofline   the dominant kernel's algorithmic bytes per launch / its average
             launch duration (HIP events on the build's stream), against the
             8 TB/s HBM peak; for the LDS-phase kernels, bound by the VALU,
             its wave64 VALU instructions per launch (rocprofv3 SQ_INSTS_VALU)
             x 64 lanes / that duration, against the 39.3 T lane-ops/s peak
  cpu_baseline  the CPU oracle on a bounded sample of the same workload

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
# kernels whose bound is the VALU (ballot ranking in LDS)
VALU_BOUND = ("k_subtree<true>", "k_subtree<false>", "k_subtree_widest")
COPY_BYTES = 256 << 20  # the --calibration-copy dispatch reads and writes this much
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def cpu_baseline(name, sample_n, widest=False):
    import oracle  # test infrastructure, used only for this reported baseline
    from tree_construction_amd import datagen
    w = datagen.WORKLOADS[name]
    pts = datagen.cached(name) if sample_n == w.n else datagen.generate(name, n=sample_n)
    oracle.load_lib()
    t0 = time.perf_counter()
    if widest:
        oracle.build_tree_widest(pts)
    else:
        oracle.build_tree(pts)
    dt = time.perf_counter() - t0
    return {"value": round(sample_n / dt / 1e6, 3), "unit": "Mpoints/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": ("the whole workload %s" % name if sample_n == w.n else
                       "same recipe and seed as %s at N=%d" % (name, sample_n))
                      + " (k=%d), %.1f s wall" % (w.k, dt)}


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
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
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


def counter_traffic(workload, kernel, widest=False):
    """Per-launch HBM bytes of `kernel` from two rocprofv3 counter runs of this
    benchmark (FETCH_SIZE, then WRITE_SIZE), each scaled by what the counter
    reads for a plain 256 MiB device copy. None if rocprofv3 is unavailable."""
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None
    out = {}
    with tempfile.TemporaryDirectory(prefix="kdt_pmc_") as tmp:
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = os.path.join(tmp, counter)
            cmd = ["timeout", "-s", "KILL", "150", prof, "--pmc", counter, "--output-format", "csv",
                   "-d", d, "-o", "kdt", "--", sys.executable, os.path.abspath(__file__),
                   "--workload", workload, "--steps", "1", "--warmup", "1", "--no-profile",
                   "--no-cpu-baseline", "--no-counters", "--calibration-copy"] + (["--widest"] if widest else [])
            r = subprocess.run(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)
            files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
            if r.returncode != 0 or not files:
                log("bench: %s counter run failed (rc %d)" % (counter, r.returncode))
                return None
            per, copy = [], []
            with open(files[0]) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    kname = kernel_short_name(row["Kernel_Name"])
                    if kname == kernel:
                        per.append(float(row["Counter_Value"]))
                    elif kname == COPY_KERNEL:
                        copy.append(float(row["Counter_Value"]))
            if not per or not copy:
                return None
            scale = (COPY_BYTES / 1024.0) / copy[0]
            out[counter] = {"bytes": sum(per) / len(per) * 1024.0 * scale, "scale": round(scale, 3)}
    return out


def counter_valu(workload, kernel, widest=False):
    """Wave64 VALU instructions per launch of `kernel` (rocprofv3 --pmc
    SQ_INSTS_VALU over one build of this benchmark), or None."""
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None
    with tempfile.TemporaryDirectory(prefix="kdt_pmc_") as tmp:
        cmd = ["timeout", "-s", "KILL", "150", prof, "--pmc", "SQ_INSTS_VALU", "--output-format", "csv",
               "-d", tmp, "-o", "kdt", "--", sys.executable, os.path.abspath(__file__),
               "--workload", workload, "--steps", "1", "--warmup", "1", "--no-profile",
               "--no-cpu-baseline", "--no-counters"] + (["--widest"] if widest else [])
        r = subprocess.run(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True)
        files = glob.glob(os.path.join(tmp, "**", "*counter_collection.csv"), recursive=True)
        if r.returncode != 0 or not files:
            log("bench: SQ_INSTS_VALU counter run failed (rc %d)" % r.returncode)
            return None
        per = []
        with open(files[0]) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == "SQ_INSTS_VALU" and kernel_short_name(row["Kernel_Name"]) == kernel:
                    per.append(float(row["Counter_Value"]))
        return sum(per) / len(per) if per else None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="points of the CPU oracle run (default: the whole workload)")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event loop")
    ap.add_argument("--no-counters", action="store_true",
                    help="skip the rocprofv3 FETCH_SIZE/WRITE_SIZE runs behind roofline.traffic")
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
                             "GBps": round(gbs, 1)}
        dom = max(kernels, key=lambda kk: kernels[kk]["ms_per_build"])
        d = kernels[dom]
        achieved = d["GBps"]
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": dom, "avg_us": d["avg_us"], "bytes_per_launch": d["bytes_per_launch"]}
        # every global sort and tag-update pass: presort histograms and passes,
        # per-round re-sorts, pivot extraction
        passes = [kk for kk in kernels if kk.startswith(("k_sort_", "k_part_", "k_pivots", "k_chunk_scan",
                                                         "k_first_digits", "k_widest_level", "k_box_"))]
        tot_b = sum(agg[kk]["bytes"] for kk in passes)
        tot_ms = sum(agg[kk]["ms"] for kk in passes)
        if tot_ms > 0:
            roofline["sort_and_update_passes"] = {
                "GBps": round(tot_b / (tot_ms * 1e-3) / 1e9, 1),
                "frac": round(tot_b / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "ms_per_build": round(tot_ms / args.steps, 4)}
        for kind, kv in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_build"]):
            log("  %-36s %4d/build  avg %8.2f us  %8.1f GB/s  %.3f ms/build"
                % (kind, kv["launches_per_build"], kv["avg_us"], kv["GBps"], kv["ms_per_build"]))
        if dom in VALU_BOUND:
            # the LDS-phase kernels rank in LDS with ballots: their bound is
            # the 32-bit VALU issue rate, not HBM
            roofline.update({"bound": "alu", "unit": "T lane-ops/s", "peak": VALU_PEAK_TLANE,
                             "achieved": None, "frac": None, "hbm_GBps": achieved})
            if not args.no_counters:
                log("bench: rocprofv3 SQ_INSTS_VALU run for %s" % dom)
                inst = counter_valu(name, dom, widest=args.widest)
                if inst:
                    lane_ops = inst * 64 / (d["avg_us"] * 1e-6) / 1e12
                    roofline.update({"achieved": round(lane_ops, 2),
                                     "frac": round(lane_ops / VALU_PEAK_TLANE, 4),
                                     "valu_instructions_per_launch": int(inst)})
                    log("  VALU %.0f M instructions per launch: %.2f T lane-ops/s (%.1f%% of %.1f)"
                        % (inst / 1e6, lane_ops, 100 * lane_ops / VALU_PEAK_TLANE, VALU_PEAK_TLANE))
        if not args.no_counters:
            log("bench: rocprofv3 FETCH_SIZE / WRITE_SIZE runs for %s" % dom)
            tr = counter_traffic(name, dom, widest=args.widest)
            if tr:
                total = tr["FETCH_SIZE"]["bytes"] + tr["WRITE_SIZE"]["bytes"]
                roofline["traffic"] = int(total)
                roofline["traffic_detail"] = {
                    "fetch_bytes": int(tr["FETCH_SIZE"]["bytes"]),
                    "write_bytes": int(tr["WRITE_SIZE"]["bytes"]),
                    "counter_scale": {"FETCH_SIZE": tr["FETCH_SIZE"]["scale"],
                                      "WRITE_SIZE": tr["WRITE_SIZE"]["scale"]},
                    "GBps": round(total / (d["avg_us"] * 1e-6) / 1e9, 1)}
                log("  traffic %s" % roofline["traffic_detail"])

    base = None
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or n
        log("bench: CPU oracle baseline on %d points" % sample)
        base = cpu_baseline(name, sample, widest=args.widest)
        log("  %s" % base)

    out = {
        "metric": ("k-d tree (split widest dimension) build Mpoints/s at N=16M k=3 fp32; achieved HBM GB/s vs peak"
                   if args.widest else "k-d tree build Mpoints/s at N=16M k=3 fp32; achieved HBM GB/s vs peak"),
        "value": round(value, 2),
        "unit": "Mpoints/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": name, "n_points": n, "k": k, "coords": "f32",
                   "description": w.note},
        "roofline": roofline,
        "cpu_baseline": base,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
