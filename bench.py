#!/usr/bin/env python3
"""Benchmark: achieved HBM bandwidth of fused residual-add + RMSNorm on MI355X.

One step = the hidden-4096 batch sweep, rows 1, 2, 4, ..., 8192 (14 launches of
norm_fused_add_rmsnorm, 16383 rows in all), over one batch of seeded synthetic
input already resident in HBM.  The value is whole-job throughput: algorithmic
bytes of the step (x and residual read, out and residual written, weight read
once per launch) divided by the step's wall time.

Steps rotate over several independent buffer sets whose total footprint is far
beyond the 256 MB Infinity Cache plus the 8 x 4 MB L2, so every step reads its
inputs from HBM (nothing is re-read warm).  Launches are replayed from HIP
graphs captured before timing (one per cycle of the buffer sets, i.e. three
steps), so the host's per-launch cost does not pace the GPU.

Also reported, on the same line:
  roofline      the dominant kernel (the kernel instantiation with the most
                GPU time in a step): its launches of a step over every buffer
                set, captured in one graph and replayed for about K steps
                between two HIP events on the launch stream; achieved =
                algorithmic bytes per launch / average launch time; beside
                it the same launches through a kernel with the same memory
                traffic and no arithmetic (libnormceiling.so): the practical
                ceiling of this traffic on the part
  kernels       the same for every instantiation the sweep uses
  sweep         per-rows GB/s, % of the 8 TB/s peak, rows/s (eager launches,
                an event pair around each, so dispatch overhead is included)
  sweep_graph   the same rows, each graph-timed on its own over enough cold
                buffer sets (time per launch includes only the GPU's gap
                between dependent launches)
  other_ops     RMSNorm / LayerNorm forward / LayerNorm backward / RMSNorm
                backward / fused add + RMSNorm backward at their largest
                workload: one graph of back-to-back launches over
                >= 1.2 GB of buffer sets (cold reads), time per launch; then
                the run-time-hidden kernels: fused add + RMSNorm at hidden
                5120 and at 4096 (forced, against the compiled kernel), an
                in-place RMSNorm over 128-wide column slices (row stride
                384), LayerNorm and RMSNorm backward at hidden 5120 and at
                32768 (rows staged in LDS); then
                few wide rows through the row-split forward (one row over
                several workgroups) beside one workgroup per row
  config_points every RMSNorm-forward and LayerNorm-forward workload point
                (hidden x rows grids of those workloads) with the kernel
                the library runs, graph-timed on cold buffers
  copy_ceiling  torch's device copy of 1 GiB, as context for the peak
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
HIDDEN = 4096
SWEEP_ROWS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)
N_SETS = 3  # 3 x 402 MB of x/residual/out buffers: no step reuses cached data
MIN_GRAPH_LAUNCHES = 18  # per-instantiation timing graphs hold at least this many launches
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def fused_bytes(rows: int, hidden: int = HIDDEN) -> int:
    return 8 * hidden * rows + 2 * hidden


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-ops", action="store_true")
    ap.add_argument("--no-hbm-ceilings", action="store_true",
                    help="skip the streaming read/write-mix ceilings (1 GiB buffers)")
    ap.add_argument("--no-config-points", action="store_true",
                    help="skip the sweep_graph and config_points legs (the counter-collection "
                         "profile runs do: rocprofv3 --pmc crashed in config_points' many "
                         "graph-replayed dispatches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="turn rocprofv3 CSV output under DIR/{stats,fetch,write} into the "
                         "summaries under profiles/ and exit (no GPU needed)")
    ap.add_argument("--profiles-out", metavar="DIR", default=PROFILES,
                    help="where --summarize-profiles writes (default: profiles/)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.profiles_out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the kernels are "
              "single-GPU and rows shard across GPUs with no communication.", file=sys.stderr)
        sys.exit(2)

    import torch
    import row_normalization_persistent_amd as rn
    from row_normalization_persistent_amd import workloads as wl

    rn.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")

    # ---- inputs: the sweep's rows concatenated; each launch gets its own slice
    total_rows = sum(SWEEP_ROWS)
    inp = wl.fused_inputs(total_rows, HIDDEN, seed=0)
    x0 = wl.to_device_bf16(inp["x"], dev)
    r0 = wl.to_device_bf16(inp["r"], dev)
    w = wl.to_device_bf16(inp["w"], dev)
    eps = inp["eps"]
    sets = []
    for _ in range(N_SETS):
        sets.append({"x": x0.clone(), "r": r0.clone(), "out": torch.empty_like(x0)})
    del x0, r0
    offs = np.cumsum((0,) + SWEEP_ROWS)
    step_bytes = sum(fused_bytes(r) for r in SWEEP_ROWS)
    cfgs = [rn.select_config("fused_add_rmsnorm", r, HIDDEN) for r in SWEEP_ROWS]
    L = rn.lib()

    stream = torch.cuda.Stream(device=dev)  # default priority
    sid = stream.cuda_stream

    def launch(s, i):
        a, b = int(offs[i]), int(offs[i + 1])
        st = L.norm_fused_add_rmsnorm(s["out"][a:b].data_ptr(), s["r"][a:b].data_ptr(),
                                      s["x"][a:b].data_ptr(), w.data_ptr(), b - a, HIDDEN,
                                      eps, sid)
        if st != 0:
            raise RuntimeError(rn.status_string(st))

    def step_eager(k):
        s = sets[k % N_SETS]
        for i in range(len(SWEEP_ROWS)):
            launch(s, i)

    # One graph per buffer set (one step each) and one graph for a whole
    # cycle of N_SETS steps (sets 0, 1, 2 in turn): K steps run as K // N_SETS
    # cycle replays plus K % N_SETS single-step replays, so the per-replay
    # submission cost is spread over N_SETS steps, as when a whole model pass
    # is captured in one graph.
    graphs = cycle = None
    if not args.no_graph:
        graphs = []
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for k in range(N_SETS):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step_eager(k)
                graphs.append(g)
            cycle = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cycle, stream=stream):
                for k in range(N_SETS):
                    step_eager(k)
        torch.cuda.synchronize()

    def run_steps(n):
        """Exactly n steps, starting at buffer set 0."""
        if graphs is None:
            for k in range(n):
                step_eager(k)
            return
        with torch.cuda.stream(stream):
            for _ in range(n // N_SETS):
                cycle.replay()
            for k in range(n % N_SETS):
                graphs[k].replay()

    # ---- warmup, then the timed region: exactly K steps
    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s over the sweep")

    # ---- per kernel instantiation: graphs holding only that instantiation's
    # launches of a step (one graph per buffer set, same row mix as the step),
    # timed with one event pair per replay on the launch stream; the dominant
    # kernel is the instantiation with the most GPU time per step
    groups = {}
    for i, c in enumerate(cfgs):
        key = _fwd_kernel_name("fused_add_rmsnorm", SWEEP_ROWS[i], HIDDEN)
        g = groups.setdefault(key, {"idx": [], "bytes": 0})
        g["idx"].append(i)
        g["bytes"] += fused_bytes(SWEEP_ROWS[i])
    def group_us_per_step(launch_fn, idx):
        """One graph walks the launches `idx` of a step over all buffer sets
        in turn, repeated until it holds at least MIN_GRAPH_LAUNCHES launches
        (so every group's per-replay cost is spread about as thinly), replayed
        about K steps' worth between two events on the launch stream: GPU
        time per step."""
        copies = max(1, -(-MIN_GRAPH_LAUNCHES // (N_SETS * len(idx))))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            cg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cg, stream=stream):
                for _ in range(copies):
                    for k in range(N_SETS):
                        for i in idx:
                            launch_fn(sets[k], i)
            cg.replay()
        reps = max(1, args.steps // N_SETS)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                cg.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        del cg
        return e0.elapsed_time(e1) * 1e3 / (reps * N_SETS * copies)

    for key, g in groups.items():
        g["us_per_step"] = group_us_per_step(launch, g["idx"])
        g["avg_launch_us"] = g["us_per_step"] / len(g["idx"])
        g["avg_bytes"] = g["bytes"] / len(g["idx"])
        g["GBps"] = g["avg_bytes"] / (g["avg_launch_us"] * 1e-6) / 1e9
    dom_key = max(groups, key=lambda k: groups[k]["us_per_step"])
    dom = groups[dom_key]
    achieved = dom["GBps"]
    kname = dom_key
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(kname, [SWEEP_ROWS[i] for i in dom["idx"]]),
                "kernel": kname, "launches_per_step": len(dom["idx"]),
                "rows_per_launch": [SWEEP_ROWS[i] for i in dom["idx"]],
                "algorithmic_bytes_per_launch": round(dom["avg_bytes"]),
                "avg_launch_us": round(dom["avg_launch_us"], 3)}
    log(f"dominant kernel {kname}: {dom['avg_launch_us']:.2f} us/launch avg, {achieved:.0f} GB/s")

    # ---- same-traffic ceiling: the dominant kernel's launches (same rows,
    # launch shapes, buffers and graph) through a kernel with its exact
    # memory traffic and no arithmetic (libnormceiling.so)
    ceil = _ceiling_fn()
    if ceil is not None and all(cfgs[i].vector_elems == 0 for i in dom["idx"]):
        def copy_launch(s, i):
            a, b = int(offs[i]), int(offs[i + 1])
            c = cfgs[i]
            st = ceil(s["out"][a:b].data_ptr(), s["r"][a:b].data_ptr(), s["x"][a:b].data_ptr(),
                      b - a, c.threads_per_row, c.rows_per_block, sid)
            if st != 0:
                raise RuntimeError(f"same-traffic kernel failed ({st}) at rows {b - a}")

        c_us = group_us_per_step(copy_launch, dom["idx"]) / len(dom["idx"])
        c_gbps = dom["avg_bytes"] / (c_us * 1e-6) / 1e9
        roofline["same_traffic_ceiling"] = {
            "kernel": "same-traffic copy: x and residual read, two outputs written, no arithmetic, "
                      "in the dominant kernel's launch shapes and row mix",
            "avg_launch_us": round(c_us, 3), "GBps": round(c_gbps, 1),
            "frac_of_peak": round(c_gbps / HBM_PEAK_GBPS, 4),
            "kernel_time_over_ceiling_time": round(dom["avg_launch_us"] / c_us, 3)}
        log(f"same-traffic ceiling: {c_us:.2f} us/launch avg, {c_gbps:.0f} GB/s")
    else:
        roofline["same_traffic_ceiling"] = None
    kernels = [{"kernel": k,
                "rows": [SWEEP_ROWS[i] for i in g["idx"]],
                "us_per_step": round(g["us_per_step"], 3),
                "avg_launch_us": round(g["avg_launch_us"], 3), "GBps": round(g["GBps"], 1)}
               for k, g in groups.items()]

    # ---- per-rows table: eager launches, each bracketed by events on the
    # launch stream (the event pair adds ~1-2 us of dispatch overhead, which
    # dominates the smallest batches)
    n_launch = len(SWEEP_ROWS)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_launch)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for k in range(args.steps):
            s = sets[k % N_SETS]
            for i in range(n_launch):
                evs[k][i][0].record(stream)
                launch(s, i)
                evs[k][i][1].record(stream)
    torch.cuda.synchronize()
    dur_us = np.array([[a.elapsed_time(b) * 1e3 for a, b in row] for row in evs])  # [K, 14]
    sweep = []
    for i, rows in enumerate(SWEEP_ROWS):
        med = float(np.median(dur_us[:, i]))
        gbps = fused_bytes(rows) / (med * 1e-6) / 1e9
        sweep.append({"rows": rows, "us_median": round(med, 3),
                      "us_p10": round(float(np.percentile(dur_us[:, i], 10)), 3),
                      "us_p90": round(float(np.percentile(dur_us[:, i], 90)), 3),
                      "GBps": round(gbps, 1), "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
                      "rows_per_s": round(rows / (med * 1e-6)),
                      "cfg": [cfgs[i].threads_per_row, cfgs[i].rows_per_block]})
        log(f"  rows {rows:5d}: {med:8.2f} us  {gbps:7.0f} GB/s  cfg {cfgs[i]}")

    result = {
        "metric": "achieved HBM GB/s (% of peak) for fused add+RMSNorm, hidden 4096, rows 1-8192",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused residual-add + RMSNorm forward, hidden 4096, one launch per "
                               "rows in {1,2,4,...,8192} per step (16383 rows), bf16 x/residual "
                               "~N(0,1), weight ~N(1,0.1), eps 1e-6, seed 0",
                   "hidden": HIDDEN, "rows": list(SWEEP_ROWS), "bytes_per_step": step_bytes,
                   "pct_peak": round(100 * value / HBM_PEAK_GBPS, 1),
                   "launch": ("hip graph replay, one graph per 3-step cycle of the buffer "
                              "sets" if graphs is not None else "eager"),
                   "buffer_sets": N_SETS},
        "roofline": roofline,
        "kernels": kernels,
        "sweep": sweep,
        "sweep_note": "eager launches with an event pair around each; includes dispatch "
                      "overhead, so small batches read low",
    }

    if not args.no_other_ops:
        result["other_ops"] = other_ops(torch, rn, wl, dev, stream,
                                        max(3, min(args.steps, 50) // 5),
                                        None if args.no_cpu_baseline else 1.0)
        if not args.no_config_points:
            result["sweep_graph"] = sweep_graph(torch, rn, dev, stream, sets[0], w, eps, offs,
                                                max(3, min(args.steps, 50) // 5))
            result["config_points"] = config_points(torch, rn, wl, dev, stream,
                                                    max(3, min(args.steps, 50) // 5))
            result["fixed_cost"] = fixed_cost(torch, rn, dev, stream, sets[0], w, eps, offs,
                                              max(3, min(args.steps, 50) // 5))
    if not args.no_hbm_ceilings:
        result["hbm_ceilings"] = hbm_ceilings(torch, dev, stream, 10)
    result["copy_ceiling"] = copy_ceiling(torch, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def load_traffic(kernel: str, rows):
    """HBM bytes per launch of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (profiles/traffic.json, written by
    `bench.py --summarize-profiles`), or None when absent, taken from a
    different kernel source, or taken over a different mix of row counts
    (the launch choice changed since)."""
    path = os.path.join(PROFILES, "traffic.json")
    try:
        t = json.load(open(path))
        entry = t["kernels"][kernel]
    except (KeyError, ValueError, OSError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    if sorted(entry.get("rows", [])) != sorted(rows):
        return None
    return round(entry["hbm_bytes_per_launch"])


def kernel_source_digest() -> str:
    """Digest of the sources that make the compiled forward kernels' code,
    comments and blank lines left out (a comment edit changes no kernel)."""
    import hashlib
    import re
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "row_normalization_persistent_amd", "csrc")
    h = hashlib.sha256()
    for name in ("device_common.hpp", "kernels_fwd.hpp", "launch.hpp"):
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()


def timed_events(torch, stream, fn, reps):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for k in range(reps):
            evs[k][0].record(stream)
            fn(k)
            evs[k][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])


def graph_time_per_launch(torch, stream, launches, reps):
    """Average time per launch of `launches` (callables, one per buffer set),
    captured in one graph and replayed `reps` times between two events."""
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for fn in launches:
                fn()
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(launches))


def _n_sets(per_set_bytes: int) -> int:
    """Buffer sets so that consecutive launches cycle through >= 1.2 GB (cold)."""
    return max(3, -(-int(1.2e9) // per_set_bytes))


def other_ops(torch, rn, wl, dev, stream, reps, cpu_seconds=None):
    """The other three operations at their largest workload: back-to-back
    launches over enough buffer sets that every launch reads cold data,
    replayed from one graph; time per launch."""
    out = []
    # RMSNorm, hidden 16384, rows 4096
    h, rows = 16384, 4096
    i = wl.rmsnorm_inputs(rows, h, seed=0)
    n = _n_sets(2 * rows * h * 2)
    x0 = wl.to_device_bf16(i["x"], dev)
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    ys = [torch.empty_like(x0) for _ in range(n)]
    w = wl.to_device_bf16(i["w"], dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_fwd(xs[j], w, i["eps"], out=ys[j], stream=stream))
        for j in range(n)], reps)
    nb = 4 * h * rows + 2 * h
    ceil = op_ceilings(torch, stream, [[xs[j]] for j in range(n)], ys, rows, h,
                       launch_shape(rn, "rmsnorm_fwd", rows, h), reps, t)
    out.append(_op_rec("rmsnorm_fwd", rows, h, nb, t, ceil=ceil,
                       cpu=oracle_beside("rmsnorm_fwd", i, rows, h, nb, cpu_seconds)))
    del xs, ys, x0
    # LayerNorm forward, hidden 16384, rows 2048
    h, rows = 16384, 2048
    i = wl.layernorm_fwd_inputs(rows, h, seed=0)
    n = _n_sets(2 * rows * h * 2)
    x0 = wl.to_device_bf16(i["x"], dev)
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    ys = [torch.empty_like(x0) for _ in range(n)]
    st = torch.empty(n, 2, rows, device=dev)
    w, bb = wl.to_device_bf16(i["w"], dev), wl.to_device_bf16(i["b"], dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.layernorm_fwd(xs[j], w, bb, i["eps"], y=ys[j], mean=st[j, 0],
                                      rstd=st[j, 1], stream=stream))
        for j in range(n)], reps)
    nb = (4 * h + 8) * rows + 4 * h
    ceil = op_ceilings(torch, stream, [[xs[j]] for j in range(n)], ys, rows, h,
                       launch_shape(rn, "layernorm_fwd", rows, h), reps, t)
    out.append(_op_rec("layernorm_fwd", rows, h, nb, t, ceil=ceil,
                       cpu=oracle_beside("layernorm_fwd", i, rows, h, nb, cpu_seconds)))
    del xs, ys, x0
    # LayerNorm backward, hidden 4096 and 8192, rows 8192
    for h in (4096, 8192):
        rows = 8192
        i = wl.layernorm_bwd_inputs(rows, h, seed=0)
        n = _n_sets(3 * rows * h * 2)
        x0 = wl.to_device_bf16(i["x"], dev)
        w = wl.to_device_bf16(i["w"], dev)
        zb = torch.zeros(h, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()  # inputs written on the current stream, used on `stream`
        _, mean, rstd = rn.layernorm_fwd(x0, w, zb, i["eps"], stream=stream)
        dy0 = wl.to_device_bf16(i["dy"], dev)
        xs = [x0] + [x0.clone() for _ in range(n - 1)]
        dys = [dy0] + [dy0.clone() for _ in range(n - 1)]
        dxs = [torch.empty_like(x0) for _ in range(n)]
        dw = torch.empty(h, device=dev)
        db = torch.empty(h, device=dev)
        ws = torch.empty(rn.workspace_bytes(rows, h), dtype=torch.uint8, device=dev)
        t = graph_time_per_launch(torch, stream, [
            (lambda j=j: rn.layernorm_bwd(dys[j], xs[j], mean, rstd, w, i["eps"], dx=dxs[j],
                                          dweight=dw, dbias=db, workspace=ws, stream=stream))
            for j in range(n)], reps)
        nb = (6 * h + 8) * rows + 10 * h
        ceil = op_ceilings(torch, stream, [[xs[j], dys[j]] for j in range(n)], dxs, rows, h,
                           launch_shape(rn, "layernorm_bwd", rows, h), reps, t)
        out.append(_op_rec("layernorm_bwd", rows, h, nb, t, ceil=ceil,
                           note="rows kernel + column-reduce kernel; workspace not counted",
                           cpu=oracle_beside("layernorm_bwd", i, rows, h, nb, cpu_seconds)))
        del xs, dys, dxs, x0, dy0
    # RMSNorm backward and the fused residual-add + RMSNorm backward, hidden 4096, rows 8192
    h, rows = 4096, 8192
    i = wl.rmsnorm_bwd_inputs(rows, h, seed=0)
    n = _n_sets(4 * rows * h * 2)
    x0, dy0, dr0 = (wl.to_device_bf16(i[k], dev) for k in ("x", "dy", "dres"))
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    dys = [dy0] + [dy0.clone() for _ in range(n - 1)]
    drs = [dr0] + [dr0.clone() for _ in range(n - 1)]
    dxs = [torch.empty_like(x0) for _ in range(n)]
    w = wl.to_device_bf16(i["w"], dev)
    dw = torch.empty(h, device=dev)
    ws = torch.empty(rn.workspace_bytes(rows, h, op="rmsnorm_bwd"), dtype=torch.uint8, device=dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_bwd(dys[j], xs[j], w, i["eps"], dx=dxs[j], dweight=dw,
                                    workspace=ws, stream=stream))
        for j in range(n)], reps)
    nb = 6 * h * rows + 6 * h
    ceil = op_ceilings(torch, stream, [[xs[j], dys[j]] for j in range(n)], dxs, rows, h,
                       launch_shape(rn, "rmsnorm_bwd", rows, h), reps, t)
    out.append(_op_rec("rmsnorm_bwd", rows, h, nb, t, ceil=ceil,
                       note="rows kernel + column-reduce kernel; workspace not counted",
                       cpu=oracle_beside("rmsnorm_bwd", i, rows, h, nb, cpu_seconds)))
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.fused_add_rmsnorm_bwd(dys[j], xs[j], w, i["eps"], dres=drs[j],
                                              ds=dxs[j], dweight=dw, workspace=ws,
                                              stream=stream))
        for j in range(n)], reps)
    nb = 8 * h * rows + 6 * h
    ceil = op_ceilings(torch, stream, [[dys[j], drs[j], xs[j]] for j in range(n)], dxs, rows, h,
                       launch_shape(rn, "fused_add_rmsnorm_bwd", rows, h), reps, t)
    out.append(_op_rec("fused_add_rmsnorm_bwd", rows, h, nb, t, ceil=ceil,
                       note="dout, dres, s read; ds written; workspace not counted",
                       cpu=oracle_beside("fused_add_rmsnorm_bwd", i, rows, h, nb,
                                         cpu_seconds)))
    del xs, dys, drs, dxs, x0, dy0, dr0
    torch.cuda.synchronize()
    out += runtime_hidden_ops(torch, rn, wl, dev, stream, reps, cpu_seconds)
    out += split_ops(torch, rn, wl, dev, stream, reps)
    out += f32_ops(torch, rn, wl, dev, stream, reps)
    return out


_CEIL_LIB = []


def _ceil_lib():
    """libnormceiling.so (the benchmark's measurement kernels, built with the
    package) with its argument types, or None when it was not built.  Loaded
    once."""
    if _CEIL_LIB:
        return _CEIL_LIB[0]
    import ctypes
    import row_normalization_persistent_amd as rn
    path = os.path.join(os.path.dirname(os.path.abspath(rn.__file__)), "libnormceiling.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.normceil_same_traffic_h4096.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    L.normceil_same_traffic_h4096.restype = ctypes.c_int
    L.normceil_stream.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i32, i64, i32,
                                  i32, vp]
    L.normceil_stream.restype = ctypes.c_int
    L.normceil_rows.argtypes = [ctypes.POINTER(vp), i32, vp, i64, i64, i32, i32, i64, i32, vp]
    L.normceil_rows.restype = ctypes.c_int
    _CEIL_LIB.append(L)
    return L


def _ceiling_fn():
    """normceil_same_traffic_h4096 from libnormceiling.so, or None."""
    L = _ceil_lib()
    return None if L is None else L.normceil_same_traffic_h4096


def launch_shape(rn, op, rows, hidden):
    """(lanes per row, 16-byte accesses per lane, persistent grid or 0, ring
    depth) of the library's launch, from its own description."""
    import re
    d = rn.describe_config(op, rows, hidden)
    lanes = int(re.search(r"\((\d+) lanes per row", d).group(1))
    vecs = int(re.search(r"(\d+) 16-byte accesses per lane", d).group(1))
    g = re.search(r"persistent grid of (\d+) workgroups", d)
    ring = re.search(r"ring of (\d+) rows", d)
    return lanes, vecs, int(g.group(1)) if g else 0, int(ring.group(1)) if ring else 1


def op_ceilings(torch, stream, ins, outs, rows, hidden, shape, reps, op_us):
    """The operation's row traffic (len(ins[j]) input matrices read, outs[j]
    written, no arithmetic) through libnormceiling.so's row kernel over the
    same buffer sets: one row per workgroup in the operation's lane layout,
    and the operation's own persistent walk (grid and ring depth) when it has
    one.  Time per launch, graph-timed like the operation; None when the
    library is not built or the layout is not compiled there."""
    import ctypes
    L = _ceil_lib()
    lanes, vecs, grid, depth = shape
    if L is None or vecs not in (1, 2, 4, 8):
        return None
    n_in = len(ins[0])
    sid = stream.cuda_stream
    ptrs = [(ctypes.c_void_p * 3)(*([t.data_ptr() for t in ins[j]] + [None] * (3 - n_in)))
            for j in range(len(outs))]
    traffic = (n_in + 1) * rows * hidden * 2

    def timed(g, d):
        def one(j):
            st = L.normceil_rows(ptrs[j], n_in, outs[j].data_ptr(), rows, hidden, lanes, vecs, g,
                                 d, sid)
            if st != 0:
                raise RuntimeError(f"normceil_rows failed ({st}) at {rows}x{hidden} "
                                   f"lanes {lanes} vecs {vecs} grid {g} depth {d}")
        one(0)  # refuses a layout it does not compile before any capture
        torch.cuda.synchronize()
        us = graph_time_per_launch(torch, stream, [(lambda j=j: one(j)) for j in
                                                   range(len(outs))], reps)
        return {"us_per_launch": round(us, 3), "GBps": round(traffic / (us * 1e-6) / 1e9, 1),
                "op_time_over_this": round(op_us / us, 3)}

    res = {"traffic_bytes": traffic,
           "reads_writes": f"{n_in} input row(s) read, 1 written, {lanes} lanes x {vecs} "
                           "16-byte accesses a row"}
    try:
        res["one_row_per_workgroup"] = timed(0, 1)
        if grid > 0:
            res["persistent_walk"] = dict(timed(grid, depth), grid=grid, depth=depth)
    except RuntimeError as e:
        log(f"  ceiling skipped: {e}")
        return None
    log(f"  same traffic: one row a workgroup {res['one_row_per_workgroup']['us_per_launch']} us"
        + (f", walk {res['persistent_walk']['us_per_launch']} us" if grid > 0 else ""))
    return res


STREAM_MIXES = (("read only", 1, 0), ("write only", 0, 1), ("copy, 1 read : 1 write", 1, 1),
                ("2 reads : 1 write", 2, 1), ("2 reads : 2 writes", 2, 2),
                ("3 reads : 1 write", 3, 1))


def hbm_ceilings(torch, dev, stream, reps):
    """The part's streaming rate for each read/write mix of the operations:
    normceil_stream over 1 GiB per buffer (so every launch streams >= 1 GiB
    through the 256 MB Infinity Cache), 16-byte non-temporal accesses, a grid
    of {1024, 2048, 4096, 8192} workgroups x {1, 2, 4, 8} accesses in flight a
    lane; the best of them per mix, time per launch over `reps` back-to-back
    launches between two events on the launch stream."""
    import ctypes
    L = _ceil_lib()
    if L is None:
        return None
    nbytes = 1 << 30
    bufs = [torch.full((nbytes // 4,), k + 1, dtype=torch.int32, device=dev) for k in range(5)]
    sink = torch.zeros(16 * 8192, dtype=torch.uint8, device=dev)
    sid = stream.cuda_stream
    out = []
    for name, nr, nw in STREAM_MIXES:
        ins = (ctypes.c_void_p * 3)(*([b.data_ptr() for b in bufs[:nr]] + [None] * (3 - nr)))
        o = [b.data_ptr() for b in bufs[3:3 + nw]] or [sink.data_ptr()]
        outs = (ctypes.c_void_p * 2)(*(o + [None] * (2 - len(o))))
        trials = []
        for grid in (1024, 2048, 4096, 8192):
            for unroll in (1, 2, 4, 8):
                def fn(k, grid=grid, unroll=unroll):
                    st = L.normceil_stream(ins, nr, outs, nw, nbytes, grid, unroll, sid)
                    if st != 0:
                        raise RuntimeError(f"normceil_stream failed ({st})")
                fn(0)
                d = timed_events(torch, stream, fn, reps)
                us = float(np.median(d))
                trials.append((us, grid, unroll))
        us, grid, unroll = min(trials)
        gbps = (nr + nw) * nbytes / (us * 1e-6) / 1e9
        out.append({"mix": name, "bytes_per_launch": (nr + nw) * nbytes, "best_grid": grid,
                    "best_accesses_in_flight": unroll, "us_median": round(us, 1),
                    "GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                    "GBps_range_over_shapes": [
                        round((nr + nw) * nbytes / (max(t[0] for t in trials) * 1e-6) / 1e9, 1),
                        round(gbps, 1)]})
        log(f"  stream {name}: {gbps:.0f} GB/s (grid {grid}, {unroll} in flight)")
    del bufs, sink
    torch.cuda.synchronize()
    return out


def sweep_graph(torch, rn, dev, stream, s0, w, eps, offs, reps):
    """Each rows value of the sweep on its own: its seeded slice of x and
    residual cloned into enough buffer sets that the graph's launches cycle
    through >= 1.2 GB, at most 512 sets (below 1 MiB a set: 256 sets, so the
    graph's submission cost is spread as thinly as at the large points; those
    few MB stay cache-resident, which latency-bound launches barely notice),
    graph-timed per launch.  The kernel-level view of the sweep (no host
    dispatch cost).  Each point also reports the same launch re-run on one
    buffer set ("warm_mall": inputs resident in the Infinity Cache), as
    context only."""
    out = []
    for i, rows in enumerate(SWEEP_ROWS):
        a, b = int(offs[i]), int(offs[i + 1])
        per_set = 8 * rows * HIDDEN
        n = min(512, _n_sets(per_set)) if per_set >= (1 << 20) else 256
        xs = [s0["x"][a:b].clone() for _ in range(n)]
        rs = [s0["r"][a:b].clone() for _ in range(n)]
        os_ = [torch.empty_like(xs[0]) for _ in range(n)]
        fns = [(lambda j=j: rn.fused_add_rmsnorm(xs[j], rs[j], w, eps, out=os_[j], stream=stream))
               for j in range(n)]
        nb = fused_bytes(rows)
        t = graph_time_per_launch(torch, stream, fns,
                                  max(2, min(reps if nb > (16 << 20) else 10 * reps, 3000 // n)))
        rec = _op_rec("fused_add_rmsnorm", rows, HIDDEN, nb, t)
        rec["rows_per_s"] = round(rows / (t * 1e-6))
        rec["kernel"] = _fwd_kernel_name("fused_add_rmsnorm", rows, HIDDEN)
        # warm (MALL): 16 launches on one buffer set, whose x, residual and out
        # (at most 192 MiB) stay in the 256 MB Infinity Cache; context only,
        # never the metric
        tw = graph_time_per_launch(torch, stream, [fns[0]] * 16,
                                   max(2, min(reps if nb > (16 << 20) else 10 * reps, 200)))
        rec["warm_mall_us"] = round(tw, 3)
        rec["warm_mall_GBps"] = round(nb / (tw * 1e-6) / 1e9, 1)
        c = rn.select_config("fused_add_rmsnorm", rows, HIDDEN)
        ceil = _ceiling_fn()
        if ceil is not None and rows >= 512 and c.vector_elems == 0:
            sid = stream.cuda_stream
            cfns = [(lambda j=j: ceil(os_[j].data_ptr(), rs[j].data_ptr(), xs[j].data_ptr(), rows,
                                      c.threads_per_row, c.rows_per_block, sid))
                    for j in range(n)]
            tc = graph_time_per_launch(torch, stream, cfns,
                                       max(2, min(reps if nb > (16 << 20) else 10 * reps,
                                                  3000 // n)))
            rec["same_traffic_us"] = round(tc, 3)
            rec["time_over_same_traffic"] = round(t / tc, 3)
        out.append(rec)
        del xs, rs, os_
    torch.cuda.synchronize()
    return out


FIXED_COST_ROWS = (1024, 2048, 4096, 8192)


def fixed_cost(torch, rn, dev, stream, s0, w, eps, offs, reps):
    """Where a fused hidden-4096 launch's time goes at 1024 ... 8192 rows: the
    library's launch beside the same launch shape (lanes per row, rows per
    workgroup, grid) doing nothing, only its reads (x and residual), only its
    writes (out and residual) and both as a plain copy (libnormceiling.so),
    each graph-timed per launch over the same cold buffer sets as sweep_graph.
    The empty grid's time is the launch's floor in a graph (dispatch and
    completion); each other figure over it is the data movement's."""
    import ctypes
    L = _ceil_lib()
    if L is None:
        return None
    L.normceil_fused_shape_part.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p]
    L.normceil_fused_shape_part.restype = ctypes.c_int
    sid = stream.cuda_stream
    out = []
    for rows in FIXED_COST_ROWS:
        i = SWEEP_ROWS.index(rows)
        a, b = int(offs[i]), int(offs[i + 1])
        n = min(512, _n_sets(8 * rows * HIDDEN))
        xs = [s0["x"][a:b].clone() for _ in range(n)]
        rs0 = [s0["r"][a:b].clone() for _ in range(n)]
        os_ = [torch.empty_like(xs[0]) for _ in range(n)]
        c = rn.select_config("fused_add_rmsnorm", rows, HIDDEN)
        if c.vector_elems != 0:
            continue
        nrep = max(2, min(reps, 3000 // n))

        def part(mode):
            def one(j):
                st = L.normceil_fused_shape_part(os_[j].data_ptr(), rs0[j].data_ptr(),
                                                 xs[j].data_ptr(), rows, c.threads_per_row,
                                                 c.rows_per_block, mode, sid)
                if st != 0:
                    raise RuntimeError(f"normceil_fused_shape_part failed ({st})")
            return graph_time_per_launch(torch, stream, [(lambda j=j: one(j)) for j in range(n)],
                                         nrep)

        t_empty, t_read, t_write = part(3), part(1), part(2)
        t_copy = graph_time_per_launch(torch, stream, [
            (lambda j=j: L.normceil_same_traffic_h4096(os_[j].data_ptr(), rs0[j].data_ptr(),
                                                       xs[j].data_ptr(), rows, c.threads_per_row,
                                                       c.rows_per_block, sid))
            for j in range(n)], nrep)
        t_op = graph_time_per_launch(torch, stream, [
            (lambda j=j: rn.fused_add_rmsnorm(xs[j], rs0[j], w, eps, out=os_[j], stream=stream))
            for j in range(n)], nrep)
        half = 4 * rows * HIDDEN
        rec = {"rows": rows, "kernel": _fwd_kernel_name("fused_add_rmsnorm", rows, HIDDEN),
               "lanes_per_row": c.threads_per_row, "rows_per_workgroup": c.rows_per_block,
               "us_empty_grid": round(t_empty, 3), "us_reads_only": round(t_read, 3),
               "us_writes_only": round(t_write, 3), "us_copy": round(t_copy, 3),
               "us_fused": round(t_op, 3),
               "GBps_reads_over_empty": round(half / ((t_read - t_empty) * 1e-6) / 1e9, 1)
               if t_read > t_empty else None,
               "GBps_writes_over_empty": round(half / ((t_write - t_empty) * 1e-6) / 1e9, 1)
               if t_write > t_empty else None,
               "pct_peak_fused": round(100 * fused_bytes(rows) / (t_op * 1e-6) / 1e9
                                       / HBM_PEAK_GBPS, 1)}
        log(f"  fixed cost {rows} rows: empty {t_empty:.2f}, reads {t_read:.2f}, writes "
            f"{t_write:.2f}, copy {t_copy:.2f}, fused {t_op:.2f} us")
        out.append(rec)
        del xs, rs0, os_
    torch.cuda.synchronize()
    return out


def config_points(torch, rn, wl, dev, stream, reps):
    """Every point of the RMSNorm-forward (hidden 2048 / 8192 / 16384 x rows
    1 / 64 / 1024 / 4096, 1 % outlier channels) and LayerNorm-forward (2048 rows
    x hidden 1024 / 4096 / 12288 / 16384) workloads, on their seeded inputs,
    with the library's launch choice: graph-timed over cold buffer sets, time
    per launch, and the kernel that runs."""
    out = []
    pts = [("rmsnorm_fwd", r, h) for h in wl.RMSNORM_HIDDEN for r in wl.RMSNORM_ROWS]
    pts += [("layernorm_fwd", wl.LAYERNORM_FWD_ROWS, h) for h in wl.LAYERNORM_FWD_HIDDEN]
    for op, rows, h in pts:
        if op == "rmsnorm_fwd":
            i = wl.rmsnorm_inputs(rows, h, seed=0)
            nb = 4 * h * rows + 2 * h
        else:
            i = wl.layernorm_fwd_inputs(rows, h, seed=0)
            nb = (4 * h + 8) * rows + 4 * h
        n = min(512, _n_sets(2 * rows * h * 2)) if rows * h * 4 >= (1 << 20) else 256
        x0 = wl.to_device_bf16(i["x"], dev)
        xs = [x0] + [x0.clone() for _ in range(n - 1)]
        ys = [torch.empty_like(x0) for _ in range(n)]
        st = torch.empty(n, 2, rows, device=dev)
        w = wl.to_device_bf16(i["w"], dev)
        if op == "rmsnorm_fwd":
            fns = [(lambda j=j: rn.rmsnorm_fwd(xs[j], w, i["eps"], out=ys[j], stream=stream))
                   for j in range(n)]
        else:
            bb = wl.to_device_bf16(i["b"], dev)
            fns = [(lambda j=j: rn.layernorm_fwd(xs[j], w, bb, i["eps"], y=ys[j], mean=st[j, 0],
                                                 rstd=st[j, 1], stream=stream))
                   for j in range(n)]
        # about 3000 launches a point at most (the small points are latency-bound)
        t = graph_time_per_launch(torch, stream, fns,
                                  max(2, min(reps if nb > (16 << 20) else 10 * reps, 3000 // n)))
        rec = _op_rec(op, rows, h, nb, t)
        rec["kernel"] = _fwd_kernel_name(op, rows, h)
        out.append(rec)
        del xs, ys, x0
    torch.cuda.synchronize()
    return out


def split_ops(torch, rn, wl, dev, stream, reps):
    """Few wide rows: the row-split forward (the library's choice of chunks)
    beside one workgroup per row, back to back from one graph over 32 buffer
    sets (a few MB: these launches are latency-bound, not bandwidth-bound)."""
    out = []
    n = 32
    ws = torch.zeros(rn.split_workspace_bytes(64), dtype=torch.uint8, device=dev)
    for op, rows, h in (("fused_add_rmsnorm", 1, 65536), ("fused_add_rmsnorm", 16, 65536),
                        ("rmsnorm_fwd", 1, 65536), ("layernorm_fwd", 1, 49152),
                        ("layernorm_fwd", 8, 65536)):
        i = (wl.fused_inputs if op == "fused_add_rmsnorm" else
             wl.rmsnorm_inputs if op == "rmsnorm_fwd" else wl.layernorm_fwd_inputs)(rows, h, 0)
        xs = [wl.to_device_bf16(i["x"], dev) for _ in range(n)]
        ys = [torch.empty_like(xs[0]) for _ in range(n)]
        w = wl.to_device_bf16(i["w"], dev)
        if op == "fused_add_rmsnorm":
            rs = [wl.to_device_bf16(i["r"], dev) for _ in range(n)]
            call = lambda j, k: rn.fused_add_rmsnorm(xs[j], rs[j], w, i["eps"], out=ys[j],
                                                     stream=stream, workspace=ws, split=k)
            nb = 8 * h * rows + 2 * h
        elif op == "rmsnorm_fwd":
            call = lambda j, k: rn.rmsnorm_fwd(xs[j], w, i["eps"], out=ys[j], stream=stream,
                                               workspace=ws, split=k)
            nb = 4 * h * rows + 2 * h
        else:
            bb = wl.to_device_bf16(i["b"], dev)
            st = torch.empty(n, 2, rows, device=dev)
            call = lambda j, k: rn.layernorm_fwd(xs[j], w, bb, i["eps"], y=ys[j], mean=st[j, 0],
                                                 rstd=st[j, 1], stream=stream, workspace=ws,
                                                 split=k)
            nb = (4 * h + 8) * rows + 4 * h
        k, v = rn.select_split(op, rows, h)
        plain = None
        if not (op == "layernorm_fwd" and h > 49152):  # one workgroup per row holds it
            plain = graph_time_per_launch(torch, stream, [
                (lambda j=j: call(j, 1)) for j in range(n)], reps)
        t = graph_time_per_launch(torch, stream, [(lambda j=j: call(j, 0)) for j in range(n)],
                                  reps)
        note = f"row split into {k} chunks of {256 * v * 8} columns"
        if plain is not None:
            note += f"; one workgroup per row: {plain:.2f} us"
        rec = _op_rec(op, rows, h, nb, t, note=note)
        rec["split"] = k
        rec["us_one_workgroup_per_row"] = None if plain is None else round(plain, 3)
        out.append(rec)
        del xs, ys
    torch.cuda.synchronize()
    return out


def runtime_hidden_ops(torch, rn, wl, dev, stream, reps, cpu_seconds=None):
    """The run-time-hidden kernels on shapes the compiled set does not cover,
    and on the headline fused shape for a like-for-like comparison with the
    compiled kernel."""
    out = []
    # fused add + RMSNorm: hidden 5120 (run-time), and hidden 4096 forced onto
    # the run-time kernels in the shape the compiled path uses there
    for h, forced in ((5120, False), (4096, True)):
        rows = 8192
        i = wl.fused_inputs(rows, h, seed=0)
        n = _n_sets(4 * rows * h * 2)
        x0, r0 = wl.to_device_bf16(i["x"], dev), wl.to_device_bf16(i["r"], dev)
        xs = [x0] + [x0.clone() for _ in range(n - 1)]
        rs = [r0] + [r0.clone() for _ in range(n - 1)]
        ys = [torch.empty_like(x0) for _ in range(n)]
        w = wl.to_device_bf16(i["w"], dev)
        cfg = None
        if forced:
            c = rn.select_config("fused_add_rmsnorm", rows, h)
            cfg = rn.Cfg(c.threads_per_row, c.rows_per_block, 0, 8)
        t = graph_time_per_launch(torch, stream, [
            (lambda j=j: rn.fused_add_rmsnorm(xs[j], rs[j], w, i["eps"], out=ys[j], cfg=cfg,
                                              stream=stream))
            for j in range(n)], reps)
        nb = 8 * h * rows + 2 * h
        out.append(_op_rec("fused_add_rmsnorm", rows, h, nb, t,
                           note="run-time-hidden kernel" + (
                               f" forced at a compiled hidden ({cfg})" if forced else ""),
                           cpu=oracle_beside("fused_add_rmsnorm", i, rows, h, nb,
                                             cpu_seconds)))
        del xs, rs, ys, x0, r0
    # RMSNorm over 128-wide head slices of a [rows, 3 * 128] projection (row
    # stride 384): the query/key normalization of a fused QKV output
    rows, h, ld = 131072, 128, 384
    i = wl.rmsnorm_inputs(rows, h, seed=0)
    n = _n_sets(rows * ld * 2)
    base0 = torch.zeros(rows, ld, dtype=torch.bfloat16, device=dev)
    base0[:, :h] = wl.to_device_bf16(i["x"], dev)
    bases = [base0] + [base0.clone() for _ in range(n - 1)]
    w = wl.to_device_bf16(i["w"], dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_fwd(bases[j][:, :h], w, i["eps"], out=bases[j][:, :h],
                                    stream=stream))
        for j in range(n)], reps)
    nb = 4 * h * rows + 2 * h
    out.append(_op_rec("rmsnorm_fwd", rows, h, nb, t,
                       note=f"in place on a column slice with row stride {ld}",
                       cpu=oracle_beside("rmsnorm_fwd", i, rows, h, nb, cpu_seconds)))
    del bases, base0
    # backward at hidden 5120 (register-resident run-time kernels) and 32768
    # (rows staged in LDS)
    for rows, h, kind in ((8192, 5120, "run-time-hidden rows kernel"),
                          (4096, 32768, "LDS-staged wide-row kernel")):
        i = wl.layernorm_bwd_inputs(rows, h, seed=0)
        n = _n_sets(3 * rows * h * 2)
        x0, dy0 = wl.to_device_bf16(i["x"], dev), wl.to_device_bf16(i["dy"], dev)
        w = wl.to_device_bf16(i["w"], dev)
        zb = torch.zeros(h, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()  # inputs written on the current stream, used on `stream`
        _, mean, rstd = rn.layernorm_fwd(x0, w, zb, i["eps"], stream=stream)
        xs = [x0] + [x0.clone() for _ in range(n - 1)]
        dys = [dy0] + [dy0.clone() for _ in range(n - 1)]
        dxs = [torch.empty_like(x0) for _ in range(n)]
        dw, db = torch.empty(h, device=dev), torch.empty(h, device=dev)
        ws = torch.empty(rn.workspace_bytes(rows, h), dtype=torch.uint8, device=dev)
        t = graph_time_per_launch(torch, stream, [
            (lambda j=j: rn.layernorm_bwd(dys[j], xs[j], mean, rstd, w, i["eps"], dx=dxs[j],
                                          dweight=dw, dbias=db, workspace=ws, stream=stream))
            for j in range(n)], reps)
        nb = (6 * h + 8) * rows + 10 * h
        ceil = op_ceilings(torch, stream, [[xs[j], dys[j]] for j in range(n)], dxs, rows, h,
                           launch_shape(rn, "layernorm_bwd", rows, h), reps, t)
        out.append(_op_rec("layernorm_bwd", rows, h, nb, t, note=kind + " + column reduce",
                           ceil=ceil,
                           cpu=oracle_beside("layernorm_bwd", i, rows, h, nb, cpu_seconds)))
        t = graph_time_per_launch(torch, stream, [
            (lambda j=j: rn.rmsnorm_bwd(dys[j], xs[j], w, wl.EPS_RMS, dx=dxs[j], dweight=dw,
                                        workspace=ws, stream=stream))
            for j in range(n)], reps)
        nb = 6 * h * rows + 6 * h
        out.append(_op_rec("rmsnorm_bwd", rows, h, nb, t, note=kind + " + column reduce",
                           cpu=oracle_beside("rmsnorm_bwd", dict(i, eps=wl.EPS_RMS), rows, h,
                                             nb, cpu_seconds)))
        del xs, dys, dxs, x0, dy0, ws
        torch.cuda.synchronize()
    out += streamed_ops(torch, rn, wl, dev, stream, reps)
    return out


def streamed_ops(torch, rn, wl, dev, stream, reps):
    """Rows no workgroup holds on chip (the streamed kernels, each row read
    twice): fused add + RMSNorm 2048 x 131072, LayerNorm forward 2048 x 65536,
    LayerNorm and RMSNorm backward 4096 x 65536; and RMSNorm 2048 x 98312 on
    the LDS-staged forward (registers and LDS, read once); time per launch over cold
    buffer sets, algorithmic bytes as for the on-chip kernels (one read and
    one write of each matrix)."""
    out = []
    h, rows = 131072, 2048
    i = wl.fused_inputs(rows, h, seed=0)
    n = _n_sets(4 * rows * h * 2)
    x0, r0 = wl.to_device_bf16(i["x"], dev), wl.to_device_bf16(i["r"], dev)
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    rs = [r0] + [r0.clone() for _ in range(n - 1)]
    ys = [torch.empty_like(x0) for _ in range(n)]
    w = wl.to_device_bf16(i["w"], dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.fused_add_rmsnorm(xs[j], rs[j], w, i["eps"], out=ys[j], stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("fused_add_rmsnorm", rows, h, 8 * h * rows + 2 * h, t,
                       note="streamed kernel: the row is read twice"))
    del xs, rs, ys, x0, r0
    h, rows = 65536, 2048
    i = wl.layernorm_fwd_inputs(rows, h, seed=0)
    n = _n_sets(2 * rows * h * 2)
    x0 = wl.to_device_bf16(i["x"], dev)
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    ys = [torch.empty_like(x0) for _ in range(n)]
    st = torch.empty(n, 2, rows, device=dev)
    w, bb = wl.to_device_bf16(i["w"], dev), wl.to_device_bf16(i["b"], dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.layernorm_fwd(xs[j], w, bb, i["eps"], y=ys[j], mean=st[j, 0],
                                      rstd=st[j, 1], stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("layernorm_fwd", rows, h, (4 * h + 8) * rows + 4 * h, t,
                       note="streamed kernel: the row is read twice"))
    del xs, ys, x0
    h, rows = 98312, 2048
    i = wl.rmsnorm_inputs(rows, h, seed=0)
    n = _n_sets(2 * rows * h * 2)
    x0 = wl.to_device_bf16(i["x"], dev)
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    ys = [torch.empty_like(x0) for _ in range(n)]
    w = wl.to_device_bf16(i["w"], dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_fwd(xs[j], w, i["eps"], out=ys[j], stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("rmsnorm_fwd", rows, h, 4 * h * rows + 2 * h, t,
                       note="LDS-staged kernel: 5 accesses a lane in registers, the rest "
                            "in LDS, the row read once"))
    del xs, ys, x0
    h, rows = 65536, 4096
    i = wl.layernorm_bwd_inputs(rows, h, seed=0)
    n = _n_sets(3 * rows * h * 2)
    x0, dy0 = wl.to_device_bf16(i["x"], dev), wl.to_device_bf16(i["dy"], dev)
    w = wl.to_device_bf16(i["w"], dev)
    zb = torch.zeros(h, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()  # inputs written on the current stream, used on `stream`
    _, mean, rstd = rn.layernorm_fwd(x0, w, zb, i["eps"], stream=stream)
    xs = [x0] + [x0.clone() for _ in range(n - 1)]
    dys = [dy0] + [dy0.clone() for _ in range(n - 1)]
    dxs = [torch.empty_like(x0) for _ in range(n)]
    dw, db = torch.empty(h, device=dev), torch.empty(h, device=dev)
    ws = torch.empty(rn.workspace_bytes(rows, h), dtype=torch.uint8, device=dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.layernorm_bwd(dys[j], xs[j], mean, rstd, w, i["eps"], dx=dxs[j],
                                      dweight=dw, dbias=db, workspace=ws, stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("layernorm_bwd", rows, h, (6 * h + 8) * rows + 10 * h, t,
                       note="streamed kernels: column tiles exchanging partial row sums "
                            "(x and dy read once) + column reduce"))
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_bwd(dys[j], xs[j], w, wl.EPS_RMS, dx=dxs[j], dweight=dw,
                                    workspace=ws, stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("rmsnorm_bwd", rows, h, 6 * h * rows + 6 * h, t,
                       note="streamed kernels: column tiles exchanging partial row sums "
                            "(x and dy read once) + column reduce"))
    drs = [torch.empty_like(x0) for _ in range(n)]
    for d in drs:
        d.copy_(dy0)
    torch.cuda.synchronize()
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.fused_add_rmsnorm_bwd(dys[j], xs[j], w, wl.EPS_RMS, dres=drs[j],
                                              ds=dxs[j], dweight=dw, workspace=ws,
                                              stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("fused_add_rmsnorm_bwd", rows, h, 8 * h * rows + 6 * h, t,
                       note="streamed kernels: column tiles exchanging partial row sums "
                            "(dout, dres and s read once) + column reduce"))
    del xs, dys, dxs, drs, x0, dy0, ws
    torch.cuda.synchronize()
    return out


def f32_ops(torch, rn, wl, dev, stream, reps):
    """fp32 activations (the `_f32` entry points) at the bf16 operations'
    configured shapes: fused add + RMSNorm 8192 x 4096, RMSNorm 4096 x 16384,
    LayerNorm forward 2048 x 16384, the three backward operations 8192 x 4096,
    and LayerNorm backward 4096 x 16384 (the LDS-staged kernel); time per
    launch over cold buffer sets, algorithmic bytes at 4 bytes an element."""
    out = []
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    def sets(a, n):
        return [a] + [a.clone() for _ in range(n - 1)]

    rows, h = 8192, 4096
    i = wl.fused_inputs(rows, h, seed=0, f32=True)
    n = _n_sets(4 * rows * h * 4)
    xs, rs = sets(f(i["x"]), n), sets(f(i["r"]), n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    w = f(i["w"])
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.fused_add_rmsnorm_f32(xs[j], rs[j], w, i["eps"], out=ys[j],
                                              stream=stream)) for j in range(n)], reps)
    out.append(_op_rec("fused_add_rmsnorm_f32", rows, h, 16 * h * rows + 4 * h, t,
                       note="fp32 activations: streamed kernel, row read once"))
    del xs, rs, ys
    rows, h = 4096, 16384
    i = wl.rmsnorm_inputs(rows, h, seed=0, f32=True)
    n = _n_sets(2 * rows * h * 4)
    xs = sets(f(i["x"]), n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    w = f(i["w"])
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_fwd_f32(xs[j], w, i["eps"], out=ys[j], stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("rmsnorm_fwd_f32", rows, h, 8 * h * rows + 4 * h, t,
                       note="fp32 activations: streamed kernel, row read once"))
    del xs, ys
    rows, h = 2048, 16384
    i = wl.layernorm_fwd_inputs(rows, h, seed=0, f32=True)
    n = _n_sets(2 * rows * h * 4)
    xs = sets(f(i["x"]), n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    st = torch.empty(n, 2, rows, device=dev)
    w, bb = f(i["w"]), f(i["b"])
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.layernorm_fwd_f32(xs[j], w, bb, i["eps"], y=ys[j], mean=st[j, 0],
                                          rstd=st[j, 1], stream=stream)) for j in range(n)],
        reps)
    out.append(_op_rec("layernorm_fwd_f32", rows, h, (8 * h + 8) * rows + 8 * h, t,
                       note="fp32 activations: streamed kernel, row read once"))
    del xs, ys
    rows, h = 8192, 4096
    i = wl.rmsnorm_bwd_inputs(rows, h, seed=0, f32=True)
    n = _n_sets(4 * rows * h * 4)
    xs, dys, drs = sets(f(i["x"]), n), sets(f(i["dy"]), n), sets(f(i["dres"]), n)
    dxs = [torch.empty_like(xs[0]) for _ in range(n)]
    w = f(i["w"])
    torch.cuda.synchronize()  # inputs written on the current stream, used on `stream`
    _, mean, rstd = rn.layernorm_fwd_f32(xs[0], w, torch.zeros_like(w), wl.EPS_LN, stream=stream)
    dw, db = torch.empty(h, device=dev), torch.empty(h, device=dev)
    ws = torch.empty(rn.workspace_bytes_f32("layernorm_bwd", rows, h), dtype=torch.uint8,
                     device=dev)
    note = ("fp32 activations: tile kernel, one 512-lane tile holds the row and reduces it "
            "(row read once) + column reduce")
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.layernorm_bwd_f32(dys[j], xs[j], mean, rstd, w, dx=dxs[j], dweight=dw,
                                          dbias=db, workspace=ws, stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("layernorm_bwd_f32", rows, h, (12 * h + 8) * rows + 12 * h, t, note=note))
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.rmsnorm_bwd_f32(dys[j], xs[j], w, i["eps"], dx=dxs[j], dweight=dw,
                                        workspace=ws, stream=stream)) for j in range(n)], reps)
    out.append(_op_rec("rmsnorm_bwd_f32", rows, h, 12 * h * rows + 8 * h, t, note=note))
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.fused_add_rmsnorm_bwd_f32(dys[j], xs[j], w, i["eps"], dres=drs[j],
                                                  ds=dxs[j], dweight=dw, workspace=ws,
                                                  stream=stream)) for j in range(n)], reps)
    out.append(_op_rec("fused_add_rmsnorm_bwd_f32", rows, h, 16 * h * rows + 8 * h, t,
                       note=note))
    del xs, dys, drs, dxs, ws
    # a row the LDS-staged backward holds (8196 ... 16384 fp32 columns)
    rows, h = 4096, 16384
    i = wl.layernorm_bwd_inputs(rows, h, seed=0, f32=True)
    n = _n_sets(3 * rows * h * 4)
    xs, dys = sets(f(i["x"]), n), sets(f(i["dy"]), n)
    dxs = [torch.empty_like(xs[0]) for _ in range(n)]
    w = f(i["w"])
    torch.cuda.synchronize()  # inputs written on the current stream, used on `stream`
    _, mean, rstd = rn.layernorm_fwd_f32(xs[0], w, torch.zeros_like(w), wl.EPS_LN, stream=stream)
    dw, db = torch.empty(h, device=dev), torch.empty(h, device=dev)
    ws = torch.empty(rn.workspace_bytes_f32("layernorm_bwd", rows, h), dtype=torch.uint8,
                     device=dev)
    t = graph_time_per_launch(torch, stream, [
        (lambda j=j: rn.layernorm_bwd_f32(dys[j], xs[j], mean, rstd, w, dx=dxs[j], dweight=dw,
                                          dbias=db, workspace=ws, stream=stream))
        for j in range(n)], reps)
    out.append(_op_rec("layernorm_bwd_f32", rows, h, (12 * h + 8) * rows + 12 * h, t,
                       note="fp32 activations: LDS-staged backward (row read once) + column "
                            "reduce"))
    del xs, dys, dxs, ws
    torch.cuda.synchronize()
    return out


def _cores():
    """(threads the oracle runs on, cores this process may run on).  The
    threads are every core in sched_getaffinity(0), capped by the host's
    per-GPU CPU share when the environment states one (OMP_NUM_THREADS: a
    host may allot a GPU's process fewer cores than the affinity mask shows)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    used = min(avail, int(share)) if share.isdigit() and int(share) > 0 else avail
    return max(1, used), max(1, avail)


def oracle_beside(op, inp, rows, hidden, nbytes, seconds):
    """The oracle on the first rows of the same workload, repeated for about
    `seconds`, as GB/s on the operation's algorithmic bytes (scaled to the
    rows timed).  Returns None when `seconds` is falsy."""
    if not seconds:
        return None
    import oracle
    cores, avail = _cores()
    k = max(1, min(rows, (1 << 22) // hidden))  # about 4 Mi elements per pass
    sl = slice(0, k)
    if op == "layernorm_bwd":
        _, mean, rstd = oracle.layernorm_fwd(inp["x"][sl], inp["w"], np.zeros(hidden, np.uint16),
                                             inp["eps"], cores)
    calls = {
        "fused_add_rmsnorm": lambda: oracle.fused_add_rmsnorm(inp["x"][sl], inp["r"][sl],
                                                              inp["w"], inp["eps"], cores),
        "rmsnorm_fwd": lambda: oracle.rmsnorm_fwd(inp["x"][sl], inp["w"], inp["eps"], cores),
        "layernorm_fwd": lambda: oracle.layernorm_fwd(inp["x"][sl], inp["w"], inp["b"],
                                                      inp["eps"], cores),
        "layernorm_bwd": lambda: oracle.layernorm_bwd(inp["dy"][sl], inp["x"][sl], mean, rstd,
                                                      inp["w"], cores),
        "rmsnorm_bwd": lambda: oracle.rmsnorm_bwd(inp["dy"][sl], inp["x"][sl], inp["w"],
                                                  inp["eps"], nthreads=cores),
        "fused_add_rmsnorm_bwd": lambda: oracle.rmsnorm_bwd(inp["dy"][sl], inp["x"][sl],
                                                            inp["w"], inp["eps"],
                                                            dres=inp["dres"][sl],
                                                            nthreads=cores),
    }
    fn = calls[op]
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        t = time.perf_counter() - t0
        if t >= seconds or reps >= 1000:
            break
    gbps = nbytes * (reps * k / rows) / t / 1e9
    return {"GBps": round(gbps, 3), "cores": cores, "cores_available": avail, "kind": "oracle",
            "sample": f"{reps} pass(es) over the first {k} of {rows} rows in {t:.2f} s"}


def _op_rec(op, rows, hidden, nbytes, us, note=None, cpu=None, ceil=None):
    gbps = nbytes / (us * 1e-6) / 1e9
    rec = {"op": op, "rows": rows, "hidden": hidden, "algorithmic_bytes": nbytes,
           "us_per_launch": round(us, 3), "GBps": round(gbps, 1),
           "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
    if note:
        rec["note"] = note
    if ceil:
        rec["same_traffic_ceiling"] = ceil
    if cpu:
        rec["cpu_oracle"] = cpu
    log(f"  {op} {rows}x{hidden}: {us:.2f} us, {gbps:.0f} GB/s"
        + (f" (oracle {cpu['GBps']} GB/s)" if cpu else ""))
    return rec


def copy_ceiling(torch, dev, stream):
    n = 1 << 29  # 512 Mi bf16 elements = 1 GiB per buffer
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    d = timed_events(torch, stream, lambda k: dst.copy_(src), 10)
    med = float(np.median(d))
    del src, dst
    return {"kernel": "torch copy_ (1 GiB read + 1 GiB write)",
            "GBps": round(2 * n * 2 / (med * 1e-6) / 1e9, 1), "us_median": round(med, 1)}


def cpu_baseline(inp, seconds):
    """The oracle (fp64 loops, C) over the same workload, repeated for about
    `seconds`; rows are split over the host cores."""
    import oracle
    cores, avail = _cores()
    x, r, w, eps = inp["x"], inp["r"], inp["w"], inp["eps"]
    offs = np.cumsum((0,) + SWEEP_ROWS)
    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while t < seconds and reps < 100:
        for i in range(len(SWEEP_ROWS)):
            a, b = int(offs[i]), int(offs[i + 1])
            oracle.fused_add_rmsnorm(x[a:b], r[a:b], w, eps, nthreads=cores)
        reps += 1
        t = time.perf_counter() - t0
    nbytes = reps * sum(fused_bytes(rr) for rr in SWEEP_ROWS)
    # the same oracle on one thread, over the sweep's rows <= 2048 (a bounded sample)
    one_rows = [rr for rr in SWEEP_ROWS if rr <= 2048]
    reps1, t1 = 0, 0.0
    t0 = time.perf_counter()
    while t1 < seconds / 2 and reps1 < 100:
        for i, rr in enumerate(SWEEP_ROWS):
            if rr <= 2048:
                a, b = int(offs[i]), int(offs[i + 1])
                oracle.fused_add_rmsnorm(x[a:b], r[a:b], w, eps, nthreads=1)
        reps1 += 1
        t1 = time.perf_counter() - t0
    nbytes1 = reps1 * sum(fused_bytes(rr) for rr in one_rows)
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": cores,
            "cores_available": avail,
            "cores_note": "threads = the cores in sched_getaffinity(0), capped by the per-GPU "
                          "CPU share the host states in OMP_NUM_THREADS",
            "kind": "oracle",
            "sample": f"{reps} pass(es) of the full rows 1..8192 sweep at hidden 4096 "
                      f"({reps * sum(SWEEP_ROWS)} rows) in {t:.1f} s",
            "one_thread": {"value": round(nbytes1 / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"{reps1} pass(es) of the sweep's rows 1..2048 "
                                     f"({reps1 * sum(one_rows)} rows) in {t1:.1f} s"}}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (profiles/)
# ---------------------------------------------------------------------------
PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats --output-format csv -d $DIR/stats -o bench -- "
    "python3 bench.py --steps 50 --warmup 5 --no-cpu-baseline --no-config-points",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $DIR/fetch -o bench -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-config-points",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $DIR/write -o bench -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-config-points",
    "rocprofv3 --pmc MeanOccupancyPerCU --output-format csv -d $DIR/occ -o bench -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-config-points",
    "rocprofv3 --pmc LdsBankConflict --output-format csv -d $DIR/lds -o bench -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-config-points",
    "python3 bench.py --summarize-profiles $DIR",
]
CALIBRATION_BYTES = 1 << 30  # the 1 GiB device copy of the copy_ceiling pass


def _short(name: str) -> str:
    return (name.replace("void ", "").replace("(anonymous namespace)::", "")
            .replace("rownorm::", "").split("(")[0])


def _tpl(name: str):
    return [int(v) for v in name.split("<")[1].split(">")[0].split(",")]


def _rows_of(name: str, grid: int):
    """Rows processed by a dispatch of one of our kernels (grid in work-items)."""
    short = _short(name).replace("_lw_kernel", "_kernel")
    if short.startswith(("fused_add_rmsnorm_kernel", "rmsnorm_fwd_kernel", "layernorm_fwd_kernel")):
        return grid // _tpl(short)[1]
    return None


def _alg_bytes(name: str, rows):
    short = _short(name).replace("_lw_kernel", "_kernel")
    if rows is None:
        return None
    h = _tpl(short)[0]
    if short.startswith("fused_add_rmsnorm_kernel"):
        return fused_bytes(rows, h)
    if short.startswith("rmsnorm_fwd_kernel"):
        return 4 * h * rows + 2 * h
    if short.startswith("layernorm_fwd_kernel"):
        return (4 * h + 8) * rows + 4 * h
    return None


# The other operations bench.py times: (op, rows, hidden, algorithmic bytes of
# the kernel that moves the rows; the backward's workspace round trip and its
# column reduce are not counted).
OTHER_WORKLOADS = [
    ("rmsnorm_fwd", 4096, 16384, lambda r, h: 4 * h * r + 2 * h),
    ("layernorm_fwd", 2048, 16384, lambda r, h: (4 * h + 8) * r + 4 * h),
    ("layernorm_bwd", 8192, 4096, lambda r, h: (6 * h + 8) * r + 2 * h),
    ("layernorm_bwd", 8192, 8192, lambda r, h: (6 * h + 8) * r + 2 * h),
    ("rmsnorm_bwd", 8192, 4096, lambda r, h: 6 * h * r + 2 * h),
    ("fused_add_rmsnorm_bwd", 8192, 4096, lambda r, h: 8 * h * r + 2 * h),
    ("fused_add_rmsnorm", 8192, 5120, lambda r, h: 8 * h * r + 2 * h),
    ("rmsnorm_fwd", 131072, 128, lambda r, h: 4 * h * r + 2 * h),
    ("layernorm_bwd", 8192, 5120, lambda r, h: (6 * h + 8) * r + 2 * h),
    ("rmsnorm_bwd", 8192, 5120, lambda r, h: 6 * h * r + 2 * h),
    ("layernorm_bwd", 4096, 32768, lambda r, h: (6 * h + 8) * r + 2 * h),
    ("rmsnorm_bwd", 4096, 32768, lambda r, h: 6 * h * r + 2 * h),
]


# The streamed and fp32 kernels bench.py times (`streamed_ops`, `f32_ops`):
# (op, rows, hidden, kernel in rocprofv3's spelling without spaces, algorithmic
# bytes of that kernel: each matrix it reads or writes once, the vectors once,
# the backward's per-row floats and partial-sum slabs not counted).
STREAM_F32_WORKLOADS = [
    ("fused_add_rmsnorm", 2048, 131072, "stream_fwd_kernel<unsignedshort,0,1024,4>",
     lambda r, h: 8 * h * r + 2 * h),
    ("layernorm_fwd", 2048, 65536, "stream_fwd_kernel<unsignedshort,2,1024,4>",
     lambda r, h: (4 * h + 8) * r + 4 * h),
    ("rmsnorm_fwd (LDS-staged)", 2048, 98312, "stage_fwd_kernel<unsignedshort,1,5,9>",
     lambda r, h: 4 * h * r + 2 * h),
    ("layernorm_bwd (tile exchange)", 4096, 65536,
     "stream_bwd_tile_kernel<unsignedshort,2,true,false,3,false,true>",
     lambda r, h: (6 * h + 8) * r + 2 * h),
    ("rmsnorm_bwd (tile exchange)", 4096, 65536,
     "stream_bwd_tile_kernel<unsignedshort,2,false,false,3,false,true>",
     lambda r, h: 6 * h * r + 2 * h),
    ("fused_add_rmsnorm_bwd (tile exchange)", 4096, 65536,
     "stream_bwd_tile_kernel<unsignedshort,2,false,true,3,false,true>",
     lambda r, h: 8 * h * r + 2 * h),
    ("fused_add_rmsnorm_f32", 8192, 4096, "stream_fwd_kernel<float,0,256,4>",
     lambda r, h: 16 * h * r + 4 * h),
    ("rmsnorm_fwd_f32", 4096, 16384, "stream_fwd_kernel<float,1,1024,4>",
     lambda r, h: 8 * h * r + 4 * h),
    ("layernorm_fwd_f32", 2048, 16384, "stream_fwd_kernel<float,2,512,8>",
     lambda r, h: (8 * h + 8) * r + 8 * h),
    ("layernorm_bwd_f32", 8192, 4096, "stream_bwd_tile_kernel<float,2,true,false,4,true,false>",
     lambda r, h: (12 * h + 8) * r + 4 * h),
    ("rmsnorm_bwd_f32", 8192, 4096, "stream_bwd_tile_kernel<float,2,false,false,4,true,false>",
     lambda r, h: 12 * h * r + 4 * h),
    ("fused_add_rmsnorm_bwd_f32", 8192, 4096,
     "stream_bwd_tile_kernel<float,2,false,true,3,true,false>",
     lambda r, h: 16 * h * r + 4 * h),
    ("layernorm_bwd_f32 (LDS-staged)", 4096, 16384, "norm_bwd_wide_kernel<float,8,true,false>",
     lambda r, h: (12 * h + 8) * r + 4 * h),
]


def _fwd_kernel_name(op, rows, hidden):
    """The forward kernel instantiation the library launches for (op, rows,
    hidden) on this device, in rocprofv3's spelling."""
    import row_normalization_persistent_amd as rn
    desc = rn.describe_config(op, rows, hidden)
    return desc.split(": ", 1)[1].split(" (", 1)[0].replace(",", ", ")


def _row_kernel_name(op, rows, hidden):
    """Kernel instantiation (rocprofv3's spelling, spaces removed) that moves
    the rows of (op, rows, hidden) with the library's own launch choice."""
    import row_normalization_persistent_amd as rn
    desc = rn.describe_config(op, rows, hidden, cu_count=256)
    k = desc.split(": ", 1)[1].split(" (", 1)[0]
    dres = "true" if op == "fused_add_rmsnorm_bwd" else "false"
    k = k.replace("norm_bwd_wide_kernel<", "norm_bwd_wide_kernel<unsignedshort,")  # element type
    return (k.replace(",layernorm>", ",true,false>").replace(",rmsnorm,dres?>", f",false,{dres}>")
             .replace(",dres?>", f",{dres}>"))


def summarize_profiles(d: str, out_dir: str = PROFILES):
    import csv
    import collections

    os.makedirs(out_dir, exist_ok=True)
    cmds = "\n".join("    " + c for c in PROFILE_COMMANDS)

    # -- kernel trace statistics
    stats = list(csv.DictReader(open(os.path.join(d, "stats", "bench_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(d, "stats", "bench_kernel_trace.csv"))))
    per = collections.defaultdict(list)
    for r in trace:
        rows = _rows_of(r["Kernel_Name"], int(r["Grid_Size_X"]))
        per[(_short(r["Kernel_Name"]), rows)].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel durations: fused residual-add + RMSNorm, hidden 4096, rows 1-8192 sweep",
             "", "Produced on one MI355X (gfx950, 256 CUs) by:", "", cmds, "",
             "`bench.py` runs the sweep from HIP graphs, then the per-instantiation graph pass "
             "behind `roofline`, the eager per-rows pass, the other operations and the "
             "1 GiB copy (every profile run skips the graph-timed per-rows sweep and the "
             "RMSNorm / LayerNorm forward workload points: they would add thousands of "
             "dispatches of the same instantiations at other row counts to the averages "
             "below).  `--stats` summary (all dispatches of the command):", "",
             "| kernel | calls | average us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "Median duration per launch size (kernel trace):", "",
              "| kernel | rows | launches | median us | GB/s (algorithmic) |",
              "|---|---:|---:|---:|---:|"]
    for (k, rows), v in sorted(per.items(), key=lambda kv: (kv[0][0], kv[0][1] or 0)):
        if rows is None:
            continue
        med = float(np.median(v))
        gbps = _alg_bytes(k, rows) / (med * 1e-6) / 1e9
        lines.append(f"| `{k}` | {rows} | {len(v)} | {med:.2f} | {gbps:.0f} |")
    lines += ["", "Launches chained in one HIP graph start as soon as their predecessor ends, "
              "so under the tracer a small launch's interval also covers the dependency wait; "
              "the large launches' intervals are their execution time."]
    open(os.path.join(out_dir, "fused_add_rmsnorm_h4096_sweep_kernel_stats.md"), "w").write(
        "\n".join(lines) + "\n")

    # -- HBM traffic from FETCH_SIZE / WRITE_SIZE (KiB per dispatch)
    def counters(sub):
        out = collections.defaultdict(list)
        calib = []
        for r in csv.DictReader(open(os.path.join(d, sub, "bench_counter_collection.csv"))):
            name = r["Kernel_Name"]
            val = float(r["Counter_Value"]) * 1024.0
            if "copyBuffer" in name:
                calib.append(val)
            rows = _rows_of(name, int(r["Grid_Size"]))
            out[(_short(name), rows)].append(val)
        return out, max(calib)
    fetch, f_cal = counters("fetch")
    write, w_cal = counters("write")
    f_scale = CALIBRATION_BYTES / f_cal
    w_scale = CALIBRATION_BYTES / w_cal
    lines = ["# HBM traffic per launch: FETCH_SIZE and WRITE_SIZE, calibrated", "",
             "Produced on one MI355X (gfx950) by:", "", cmds, "",
             f"Calibration: the 1 GiB device-to-device copy in `bench.py` (1 GiB read, 1 GiB "
             f"written) reads FETCH_SIZE = {f_cal / 2**20:.1f} MiB and WRITE_SIZE = "
             f"{w_cal / 2**20:.1f} MiB, so FETCH_SIZE is scaled by {f_scale:.4f} and "
             f"WRITE_SIZE by {w_scale:.4f}.", "",
             "| kernel | rows | dispatches | read MiB (scaled) | written MiB (scaled) | "
             "algorithmic MiB | HBM / algorithmic |", "|---|---:|---:|---:|---:|---:|---:|"]
    kernels = {}
    groups = collections.defaultdict(lambda: {"hbm": [], "alg": [], "rows": []})
    for key in sorted(set(fetch) & set(write), key=lambda k: (k[0], k[1] or 0)):
        k, rows = key
        if not k.startswith(("fused_add", "rmsnorm", "layernorm")):
            continue
        rd = float(np.mean(fetch[key])) * f_scale
        wr = float(np.mean(write[key])) * w_scale
        alg = _alg_bytes(k, rows)
        ratio = f"{(rd + wr) / alg:.4f}" if alg else "-"
        algs = f"{alg / 2**20:.2f}" if alg else "-"
        lines.append(f"| `{k}` | {rows if rows is not None else '-'} | {len(fetch[key])} | "
                     f"{rd / 2**20:.2f} | {wr / 2**20:.2f} | {algs} | {ratio} |")
        if alg:
            n = min(len(fetch[key]), len(write[key]))
            groups[k]["hbm"] += [rd + wr] * n
            groups[k]["alg"] += [alg] * n
            groups[k]["rows"].append(rows)
    for k, g in groups.items():
        kernels[k] = {"hbm_bytes_per_launch": float(np.mean(g["hbm"])),
                      "algorithmic_bytes_per_launch": float(np.mean(g["alg"])),
                      "rows": sorted(g["rows"])}
    lines += ["", "The other operations (`other_ops`), kernel that moves the rows, algorithmic bytes "
              "without the backward workspace (its round trip shows as the excess):", "",
              "| op | rows x hidden | kernel | dispatches | read MiB | written MiB | "
              "algorithmic MiB | HBM / algorithmic |", "|---|---|---|---:|---:|---:|---:|---:|"]
    by_name = collections.defaultdict(lambda: ([], []))
    for (k, _rows), v in fetch.items():
        by_name[k.replace(" ", "")][0].extend(v)
    for (k, _rows), v in write.items():
        by_name[k.replace(" ", "")][1].extend(v)
    for op, rows, h, alg_fn in OTHER_WORKLOADS:
        try:
            kname = _row_kernel_name(op, rows, h)
        except Exception:  # the library is not built here: skip the table
            break
        f_v, w_v = by_name.get(kname, ([], []))
        if not f_v or not w_v:
            continue
        rd = float(np.mean(f_v)) * f_scale
        wr = float(np.mean(w_v)) * w_scale
        alg = alg_fn(rows, h)
        lines.append(f"| {op} | {rows} x {h} | `{kname}` | {len(f_v)} | {rd / 2**20:.2f} | "
                     f"{wr / 2**20:.2f} | {alg / 2**20:.2f} | {(rd + wr) / alg:.4f} |")
    stream_f32 = []
    for op, rows, h, kname, alg_fn in STREAM_F32_WORKLOADS:
        f_v, w_v = by_name.get(kname, ([], []))
        if not f_v or not w_v:
            continue
        rd = float(np.mean(f_v)) * f_scale
        wr = float(np.mean(w_v)) * w_scale
        alg = alg_fn(rows, h)
        stream_f32.append(f"| {op} | {rows} x {h} | `{kname}` | {len(f_v)} | {rd / 2**20:.2f} | "
                          f"{wr / 2**20:.2f} | {alg / 2**20:.2f} | {(rd + wr) / alg:.4f} |")
    if stream_f32:
        lines += ["", "The streamed kernels (`streamed_ops`: rows past the on-chip kernels, each "
                  "row read twice) and the fp32-activation kernels (`f32_ops`), algorithmic bytes "
                  "counting each matrix once (a streamed row's second read shows as the excess "
                  "when it misses the Infinity Cache):", "",
                  "| op | rows x hidden | kernel | dispatches | read MiB | written MiB | "
                  "algorithmic MiB | HBM / algorithmic |", "|---|---|---|---:|---:|---:|---:|---:|"]
        lines += stream_f32
    # the streaming ceilings move known bytes (1 GiB per buffer): their scaled
    # counters check the calibration and the kernels' own traffic
    import re as _re
    stream_rows = []
    for (k, _rows), v in sorted(fetch.items()):
        m = _re.search(r"stream_kernel<(\d+), (\d+), (\d+)>", k)
        if not m or (k, _rows) not in write:
            continue
        nr, nw, u = (int(g) for g in m.groups())
        rd = float(np.mean(v)) * f_scale
        wr = float(np.mean(write[(k, _rows)])) * w_scale
        exp_r, exp_w = nr * CALIBRATION_BYTES, nw * CALIBRATION_BYTES
        stream_rows.append(f"| {nr} : {nw} | {u} | {len(v)} | {rd / 2**20:.1f} | "
                           f"{exp_r / 2**20:.0f} | {wr / 2**20:.1f} | {exp_w / 2**20:.0f} |")
    if stream_rows:
        lines += ["", "The streaming ceilings (`hbm_ceilings`, `normceil_stream` over 1 GiB "
                  "buffers: reads : writes, accesses in flight a lane) against the bytes they "
                  "touch, averaged over their dispatches (every grid size of the sweep):", "",
                  "| reads : writes | in flight | dispatches | read MiB (scaled) | buffers read "
                  "MiB | written MiB (scaled) | buffers written MiB |",
                  "|---|---:|---:|---:|---:|---:|---:|"] + stream_rows
    lines += ["", "Per-launch averages over each kernel's dispatches (the mix of row counts "
              "the sweep gives it) are in `profiles/traffic.json`, which `bench.py` reports as "
              "`roofline.traffic` while the kernel sources and the kernel's mix of row counts are "
              "unchanged."]
    open(os.path.join(out_dir, "fused_add_rmsnorm_h4096_sweep_hbm_traffic.md"), "w").write(
        "\n".join(lines) + "\n")
    json.dump({"kernel_source_sha256": kernel_source_digest(),
               "fetch_scale": f_scale, "write_scale": w_scale, "kernels": kernels},
              open(os.path.join(out_dir, "traffic.json"), "w"), indent=1)

    # -- occupancy and LDS bank conflicts (rocprofv3 derived counters), when collected
    if os.path.isdir(os.path.join(d, "occ")) and os.path.isdir(os.path.join(d, "lds")):
        res = {}  # kernel -> (VGPRs per lane, LDS bytes per workgroup, workgroup size)

        def derived(sub, name):
            out = collections.defaultdict(list)
            for r in csv.DictReader(open(os.path.join(d, sub, "bench_counter_collection.csv"))):
                if r["Counter_Name"] == name:
                    k = _short(r["Kernel_Name"])
                    out[k].append(float(r["Counter_Value"]))
                    res[k] = (r["VGPR_Count"], r["LDS_Block_Size"], r["Workgroup_Size"])
            return out
        occ = derived("occ", "MeanOccupancyPerCU")
        lds = derived("lds", "LdsBankConflict")
        lines = ["# Occupancy and LDS bank conflicts per kernel", "",
                 "Produced on one MI355X (gfx950, 256 CUs) by:", "", cmds, "",
                 "`MeanOccupancyPerCU` is rocprofv3's derived counter: resident waves summed "
                 "over the dispatch's busy cycles, divided by those cycles and by the CU count "
                 "(a CU holds at most 32 waves here: 8 per SIMD).  `LdsBankConflict` is "
                 "SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT): cycles lost "
                 "to bank conflicts per conflict-free LDS cycle (0 = none).  Averages over each "
                 "kernel's dispatches in the profiled command; short launches are dominated by "
                 "their ramp, so their occupancy reads low.", "",
                 "| kernel | workgroup | VGPR_Count (as rocprofv3 reports it) | LDS bytes | "
                 "dispatches | mean waves per CU | "
                 "LDS conflict cycles per LDS cycle |", "|---|---:|---:|---:|---:|---:|---:|"]
        for k in sorted(set(occ) | set(lds)):
            if not k.startswith(("fused_add", "rmsnorm", "layernorm", "norm_", "split_")):
                continue
            o = f"{np.mean(occ[k]):.2f}" if occ.get(k) else "-"
            c = f"{np.mean(lds[k]):.4f}" if lds.get(k) else "-"
            wg, vg, lb = res[k][2], res[k][0], res[k][1]
            lines.append(f"| `{k}` | {wg} | {vg} | {lb} | "
                         f"{max(len(occ.get(k, [])), len(lds.get(k, [])))} | {o} | {c} |")
        open(os.path.join(out_dir, "fused_add_rmsnorm_h4096_sweep_occupancy_lds.md"), "w").write(
            "\n".join(lines) + "\n")
    print(f"wrote summaries to {out_dir}")


if __name__ == "__main__":
    main()
