"""bench.py's profile summarisers on hand-made rocprofv3-shaped CSV files (the
column names of rocprofv3's kernel_trace / kernel_stats / counter_collection
outputs): runs of dispatches split at idle gaps, the counter table's byte
calibration, clock, L2 hit rate and per-call traffic, worked out by hand for
the numbers below; and the refusal to write a summary without its commands."""
from __future__ import annotations

import csv
import json
import os
import re

import pytest

import bench

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp"]
STATS_COLS = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
              "StdDev"]
COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
                "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_csv(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=cols)
        wr.writeheader()
        for r in rows:
            wr.writerow({c: r.get(c, 0) for c in cols})


def test_trace_runs_split_at_idle_gaps(tmp_path):
    d = tmp_path / "trace"
    rows, t = [], 1_000_000_000
    # kernel A: 6 dispatches of 100 us, 1 s idle, 5 dispatches of 200 us; kernel B in between
    for i in range(6):
        rows.append({"Dispatch_Id": i, "Kernel_Name": "kA", "Start_Timestamp": t,
                     "End_Timestamp": t + 100_000})
        t += 110_000
    rows.append({"Dispatch_Id": 6, "Kernel_Name": "kB", "Start_Timestamp": t,
                 "End_Timestamp": t + 5_000})
    t += 1_000_000_000
    for i in range(5):
        rows.append({"Dispatch_Id": 7 + i, "Kernel_Name": "kA", "Start_Timestamp": t,
                     "End_Timestamp": t + 200_000})
        t += 210_000
    _write_csv(str(d / "x_kernel_trace.csv"), TRACE_COLS, rows)
    _write_csv(str(d / "x_kernel_stats.csv"), STATS_COLS,
               [{"Name": "kA", "Calls": 11, "AverageNs": 145454.5, "Percentage": 99.0,
                 "MinNs": 100000, "MaxNs": 200000}])
    runs = bench._dispatch_runs(list(csv.DictReader(open(d / "x_kernel_trace.csv"))))
    assert [(k, len(dur)) for k, dur, _ in runs] == [("kA", 6), ("kB", 1), ("kA", 5)]
    assert runs[0][1][0] == 100.0 and runs[2][1][0] == 200.0
    out = tmp_path / "s.md"
    bench.summarize_trace(str(d), str(out), "rocprofv3 --kernel-trace --stats -- python3 bench.py")
    text = out.read_text()
    assert "| 1 | `kA` | 6 | 100.0 |" in text and "| 2 | `kA` | 5 | 200.0 |" in text
    assert "rocprofv3 --kernel-trace --stats -- python3 bench.py" in text


def test_counter_summary_by_hand(tmp_path):
    # the calibration copy: 256 MiB each way, FETCH_SIZE reads half, WRITE_SIZE all
    kib = 256 * 1024
    gemm = "void g355::gemm_f32_ring_kernel<256, 256, 3, 2, 4, 8, false, false>(g355::F32Args)"
    copy = "g355::(anonymous namespace)::copy_f32_kernel(float4 const*, float4*, long)"
    dirs = []
    counters = [  # pass 1: utilisations and the clock counter; pass 2: L2 and writes; pass 3: fetch
        {gemm: {"MfmaUtil": 90.0, "LdsBankConflict": 0.01, "LdsUtil": 30.0,
                "GRBM_GUI_ACTIVE": 8 * 2000.0 * 1000.0}},       # 2000 MHz x 1000 us, 8 XCDs
        {gemm: {"TCC_HIT_sum": 900.0, "TCC_MISS_sum": 100.0, "WRITE_SIZE": 65536.0},
         copy: {"WRITE_SIZE": float(kib)}},
        {gemm: {"FETCH_SIZE": 98304.0}, copy: {"FETCH_SIZE": kib / 2.0}},
    ]
    for p, kernels in enumerate(counters):
        d = tmp_path / f"pass{p}"
        crow, trow = [], []
        for disp, (name, vals) in enumerate(kernels.items()):
            for c, v in vals.items():
                crow.append({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c,
                             "Counter_Value": v})
            dur = 1_000_000 if name == gemm else 50_000     # ns
            trow.append({"Dispatch_Id": disp, "Kernel_Name": name, "Start_Timestamp": 10,
                         "End_Timestamp": 10 + dur})
        _write_csv(str(d / "r_counter_collection.csv"), COUNTER_COLS, crow)
        _write_csv(str(d / "r_kernel_trace.csv"), TRACE_COLS, trow)
        dirs.append(str(d))
    out = tmp_path / "c.md"
    with pytest.raises(SystemExit):
        bench.summarize_counters("f32_4096_a1_b0", dirs, str(out), "")
    bench.summarize_counters("f32_4096_a1_b0", dirs, str(out), "rocprofv3 --pmc ... (3 passes)")
    text = out.read_text()
    meta = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    k = meta["kernels"][gemm]
    assert k["clock_mhz"] == pytest.approx(2000.0)
    assert k["cycles_per_xcd"] == pytest.approx(2000.0 * 1000.0)
    assert meta["tile"].startswith("BM=")
    assert k["l2_hit"] == pytest.approx(0.9)
    assert k["mfma_util_pct"] == 90.0 and k["lds_bank_conflict_per_access"] == 0.01
    # fetch 98304 KiB x 2 = 192 MiB read; write 65536 KiB x 1 = 64 MiB
    assert k["hbm_read_bytes"] == pytest.approx(192 * 2 ** 20)
    assert k["hbm_write_bytes"] == pytest.approx(64 * 2 ** 20)
    assert meta["traffic_bytes_per_call"] == pytest.approx(256 * 2 ** 20)
    # compulsory at 4096^3, beta = 0: 4(MK + KN) + 4MN = 3 x 64 MiB
    assert meta["compulsory_bytes"] == pytest.approx(3 * 64 * 2 ** 20)
    assert meta["fetch_factor"] == pytest.approx(2.0) and meta["write_factor"] == pytest.approx(1.0)


def test_profile_target_names_a_workload_or_a_shape():
    w = bench.profile_target("f32_4096_a1_b1")
    assert (w.mode, w.M, w.N, w.K, w.beta) == ("f32", 4096, 4096, 4096, 1.0)
    s = bench.profile_target("f16r:128x4096x2048")
    assert (s.mode, s.M, s.N, s.K, s.alpha, s.beta) == ("f16r", 128, 4096, 2048, 1.0, 0.0)
    for bad in ("f64:1x2x3", "f32:1x2", "nothing"):
        with pytest.raises(SystemExit):
            bench.profile_target(bad)
