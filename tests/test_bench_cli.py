"""bench.py host-side behaviour (CPU only): the one-GPU guard and the
rocprofv3 summary arithmetic (FETCH_SIZE / WRITE_SIZE calibration) and when the
recorded traffic applies."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")
K = "void rownorm::fused_add_rmsnorm_kernel<4096, 128, 2>(unsigned int __vector(4)*, long, float)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_calibrates_counters(tmp_path):
    d = tmp_path / "prof"
    _write(str(d / "stats" / "bench_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"], [[K, 2, 80000, 40000.0, 100.0, 39000, 41000, 1.0]])
    trace_hdr = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id",
                 "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp",
                 "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                 "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y",
                 "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    _write(str(d / "stats" / "bench_kernel_trace.csv"), trace_hdr,
           [["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i, 7, K, i, 1000, 1000 + 40000, 0, 0, 80, 0,
             20, 256, 1, 1, 8192 * 128, 1, 1] for i in range(2)])
    pmc_hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
               "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
               "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
               "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    gib_kib = float(1 << 20)
    # the copy reads half of what it moves on FETCH_SIZE (scale 2), all on WRITE_SIZE
    _write(str(d / "fetch" / "bench_counter_collection.csv"), pmc_hdr,
           [[1, 1, "Agent 1", 1, 1, 1, 131072, 8, "__amd_rocclr_copyBuffer", 512, 0, 0, 8, 0, 32,
             "FETCH_SIZE", gib_kib / 2, 0, 1],
            [2, 2, "Agent 1", 1, 1, 1, 8192 * 128, 7, K, 256, 0, 0, 80, 0, 20, "FETCH_SIZE",
             65536.0, 0, 1]])
    _write(str(d / "write" / "bench_counter_collection.csv"), pmc_hdr,
           [[1, 1, "Agent 1", 1, 1, 1, 131072, 8, "__amd_rocclr_copyBuffer", 512, 0, 0, 8, 0, 32,
             "WRITE_SIZE", gib_kib, 0, 1],
            [2, 2, "Agent 1", 1, 1, 1, 8192 * 128, 7, K, 256, 0, 0, 80, 0, 20, "WRITE_SIZE",
             131072.0, 0, 1]])
    out = tmp_path / "out"
    r = subprocess.run([sys.executable, BENCH, "--summarize-profiles", str(d), "--profiles-out",
                        str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    t = json.load(open(out / "traffic.json"))
    assert abs(t["fetch_scale"] - 2.0) < 1e-12 and abs(t["write_scale"] - 1.0) < 1e-12
    k = t["kernels"]["fused_add_rmsnorm_kernel<4096, 128, 2>"]
    assert k["rows"] == [8192]
    assert k["hbm_bytes_per_launch"] == 2 * 65536 * 1024 + 131072 * 1024
    assert k["algorithmic_bytes_per_launch"] == 8 * 4096 * 8192 + 2 * 4096
    md = open(out / "fused_add_rmsnorm_h4096_sweep_kernel_stats.md").read()
    assert "rocprofv3 --kernel-trace --stats" in md and "| 8192 | 2 | 40.00 |" in md


def test_traffic_is_reported_only_for_the_profiled_kernel_and_row_mix(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    kname = "fused_add_rmsnorm_kernel<4096, 128, 2>"
    rec = {"kernel_source_sha256": bench.kernel_source_digest(),
           "kernels": {kname: {"hbm_bytes_per_launch": 1234.4, "rows": [512, 4096, 8192]}}}
    json.dump(rec, open(tmp_path / "traffic.json", "w"))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic(kname, [8192, 512, 4096]) == 1234
    assert bench.load_traffic(kname, [4096, 8192]) is None        # launch choice changed
    assert bench.load_traffic("fused_add_rmsnorm_kernel<4096, 64, 4>", [1024]) is None
    rec["kernel_source_sha256"] = "0" * 64                       # kernel code changed
    json.dump(rec, open(tmp_path / "traffic.json", "w"))
    assert bench.load_traffic(kname, [512, 4096, 8192]) is None
