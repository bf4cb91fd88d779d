#!/usr/bin/env python3
"""Benchmark: achieved HBM bandwidth of fused residual-add + RMSNorm on MI355X.

One step = the hidden-4096 batch sweep, rows 1, 2, 4, ..., 8192 (14 launches of
norm_fused_add_rmsnorm, 16383 rows in all), over one batch of seeded synthetic
input already resident in HBM.  The value is whole-job throughput: algorithmic
bytes of the step (x and residual read, out and residual written, weight read
once per launch) divided by the step's wall time.

Steps rotate over several independent buffer sets whose total footprint is far
beyond the 256 MB Infinity Cache plus the 8 x 4 MB L2, so every step reads its
inputs from HBM (nothing is re-read warm).  Launches are replayed from one HIP
graph per buffer set (captured once, before timing), so the host's per-launch
cost does not pace the GPU.

Also reported, on the same line:
  roofline      the dominant kernel (the kernel instantiation with the most
                GPU time in a step), timed with HIP events on its own stream
                over a second timed pass of the same launches
  sweep         per-rows achieved GB/s, % of the 8 TB/s peak, rows/s
  other_ops     RMSNorm / LayerNorm forward / LayerNorm backward at their
                largest workload, GB/s by the same rule
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
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
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

    graphs = None
    if not args.no_graph:
        graphs = []
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for k in range(N_SETS):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step_eager(k)
                graphs.append(g)
        torch.cuda.synchronize()

    def step(k):
        if graphs is not None:
            with torch.cuda.stream(stream):
                graphs[k % N_SETS].replay()
        else:
            step_eager(k)

    # ---- warmup, then the timed region: exactly K steps
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s over the sweep")

    # ---- second timed pass: every launch bracketed by events on its stream
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

    # dominant kernel: the instantiation with the most GPU time per step
    groups = {}
    for i, c in enumerate(cfgs):
        key = (c.threads_per_row, c.rows_per_block)
        g = groups.setdefault(key, {"idx": [], "bytes": 0})
        g["idx"].append(i)
        g["bytes"] += fused_bytes(SWEEP_ROWS[i])
    dom_key = max(groups, key=lambda k: dur_us[:, groups[k]["idx"]].sum())
    dom = groups[dom_key]
    n_dom = len(dom["idx"])
    avg_dur = float(dur_us[:, dom["idx"]].sum() / (args.steps * n_dom))
    avg_bytes = dom["bytes"] / n_dom
    achieved = avg_bytes / (avg_dur * 1e-6) / 1e9
    kname = f"fused_add_rmsnorm_kernel<{HIDDEN}, {dom_key[0]}, {dom_key[1]}>"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(kname, avg_bytes),
                "kernel": kname, "launches_per_step": n_dom,
                "rows_per_launch": [SWEEP_ROWS[i] for i in dom["idx"]],
                "algorithmic_bytes_per_launch": round(avg_bytes),
                "avg_launch_us": round(avg_dur, 3)}
    log(f"dominant kernel {kname}: {avg_dur:.2f} us/launch avg, {achieved:.0f} GB/s")

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
                   "launch": "hip graph replay" if graphs is not None else "eager",
                   "buffer_sets": N_SETS},
        "roofline": roofline,
        "sweep": sweep,
    }

    if not args.no_other_ops:
        result["other_ops"] = other_ops(torch, rn, wl, dev, stream, min(args.steps, 50))
    result["copy_ceiling"] = copy_ceiling(torch, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def load_traffic(kernel: str, alg_bytes: float):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    scaled by the copy-kernel calibration; None when absent or stale."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
        entry = t["kernels"][kernel]
    except (KeyError, ValueError):
        return None
    if entry.get("source_sha256") != kernel_source_digest():
        return None
    return round(entry["bytes_per_launch"])


def kernel_source_digest() -> str:
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "row_normalization_persistent_amd", "csrc")
    h = hashlib.sha256()
    for name in ("device_common.hpp", "kernels_fwd.hpp"):
        h.update(open(os.path.join(csrc, name), "rb").read())
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


def other_ops(torch, rn, wl, dev, stream, reps):
    """The other three operations at their largest workload, cold buffers."""
    out = []
    nset = 3
    # RMSNorm, hidden 16384, rows 4096
    h, rows = 16384, 4096
    i = wl.rmsnorm_inputs(rows, h, seed=0)
    xs = [wl.to_device_bf16(i["x"], dev) for _ in range(nset)]
    os_ = [torch.empty_like(xs[0]) for _ in range(nset)]
    w = wl.to_device_bf16(i["w"], dev)
    for k in range(3):
        rn.rmsnorm_fwd(xs[k % nset], w, i["eps"], out=os_[k % nset], stream=stream)
    d = timed_events(torch, stream,
                     lambda k: rn.rmsnorm_fwd(xs[k % nset], w, i["eps"], out=os_[k % nset],
                                              stream=stream), reps)
    b = 4 * h * rows + 2 * h
    out.append(_op_rec("rmsnorm_fwd", rows, h, b, d))
    del xs, os_
    # LayerNorm forward, hidden 16384, rows 2048
    h, rows = 16384, 2048
    i = wl.layernorm_fwd_inputs(rows, h, seed=0)
    xs = [wl.to_device_bf16(i["x"], dev) for _ in range(nset)]
    ys = [torch.empty_like(xs[0]) for _ in range(nset)]
    ms = [torch.empty(rows, device=dev) for _ in range(nset)]
    rs = [torch.empty(rows, device=dev) for _ in range(nset)]
    w, bb = wl.to_device_bf16(i["w"], dev), wl.to_device_bf16(i["b"], dev)

    def lnf(k):
        j = k % nset
        rn.layernorm_fwd(xs[j], w, bb, i["eps"], y=ys[j], mean=ms[j], rstd=rs[j], stream=stream)
    for k in range(3):
        lnf(k)
    d = timed_events(torch, stream, lnf, reps)
    out.append(_op_rec("layernorm_fwd", rows, h, (4 * h + 8) * rows + 4 * h, d))
    del xs, ys
    # LayerNorm backward, hidden 4096 and 8192, rows 8192
    for h in (4096, 8192):
        rows = 8192
        i = wl.layernorm_bwd_inputs(rows, h, seed=0)
        x = wl.to_device_bf16(i["x"], dev)
        w = wl.to_device_bf16(i["w"], dev)
        zb = torch.zeros(h, dtype=torch.bfloat16, device=dev)
        _, mean, rstd = rn.layernorm_fwd(x, w, zb, i["eps"], stream=stream)
        xs = [x] + [x.clone() for _ in range(nset - 1)]
        dys = [wl.to_device_bf16(i["dy"], dev) for _ in range(nset)]
        dxs = [torch.empty_like(x) for _ in range(nset)]
        dw = torch.empty(h, device=dev)
        db = torch.empty(h, device=dev)
        ws = torch.empty(rn.workspace_bytes(rows, h), dtype=torch.uint8, device=dev)

        def lnb(k):
            j = k % nset
            rn.layernorm_bwd(dys[j], xs[j], mean, rstd, w, i["eps"], dx=dxs[j], dweight=dw,
                             dbias=db, workspace=ws, stream=stream)
        for k in range(3):
            lnb(k)
        d = timed_events(torch, stream, lnb, reps)
        out.append(_op_rec("layernorm_bwd", rows, h, (6 * h + 8) * rows + 10 * h, d,
                           note="rows kernel + column-reduce kernel; workspace not counted"))
        del xs, dys, dxs
    torch.cuda.synchronize()
    return out


def _op_rec(op, rows, hidden, nbytes, d, note=None):
    med = float(np.median(d))
    gbps = nbytes / (med * 1e-6) / 1e9
    rec = {"op": op, "rows": rows, "hidden": hidden, "algorithmic_bytes": nbytes,
           "us_median": round(med, 3), "GBps": round(gbps, 1),
           "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)}
    if note:
        rec["note"] = note
    log(f"  {op} {rows}x{hidden}: {med:.2f} us, {gbps:.0f} GB/s")
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
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
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
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} pass(es) of the full rows 1..8192 sweep at hidden 4096 "
                      f"({reps * sum(SWEEP_ROWS)} rows) in {t:.1f} s"}


if __name__ == "__main__":
    main()
