"""bench.py's output contract on a short run: one JSON line on stdout's last
line with the headline fields, a roofline object whose fraction is
achieved / peak, and the oracle's CPU baseline beside it.  The bench runs as a
child process (a fresh HIP context), cut to a few steps and a 1 s CPU sample."""
import json
import os
import subprocess
import sys
import time

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    t0 = time.time()
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--no-other-ops", "--no-config-points", "--cpu-seconds", "1"]
    out = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=100)
    print(f"bench took {time.time() - t0:.1f} s", flush=True)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert sum(ln.lstrip().startswith("{") for ln in lines) == 1, "exactly one JSON line"
    d = json.loads(lines[-1])
    assert d["metric"].startswith("achieved HBM GB/s (% of peak) for fused add+RMSNorm")
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["dtype"] == "bf16" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert d["scaling"] in ("weak", "strong")
    assert 0 < d["value"] < 8000 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] < r["peak"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert c["unit"] == "GB/s" and c["sample"]
