"""Host logic of bench.py that turns rocprofv3 output into the committed
summaries (CPU only): the traffic summary's launch selection and scaling,
and the trace summary's runs."""
import csv
import io
import json
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FUSED = "void tq::(anonymous namespace)::%s(unsigned char const*, ...)" % bench.TRAFFIC_KERNEL
DOWN = "void tq::(anonymous namespace)::gemv_xreg_kernel<0, 64, 4, 8, false, true, 16>(...)"
COPY = "__amd_rocclr_copyBuffer"


def write_counters(path, rows, counter):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, grid, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Grid_Size": grid, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": value})


def test_traffic_json_selects_fused_launches_and_scales(tmp_path):
    # 7 fused launches (about 23250 KiB each), unfused gate launches of the
    # same template and grid at half the bytes, and down launches
    fetch = [(FUSED, "131072", 23250.0)] * 7 + [(FUSED, "131072", 11700.0)] * 4 + [(DOWN, "131072", 11600.0)] * 5
    write = [(FUSED, "131072", 136.0)] * 7 + [(FUSED, "131072", 68.0)] * 4 + [(DOWN, "131072", 20.0)] * 5
    cal_f = [(COPY, "131072", 524288.0)] * 3
    cal_w = [(COPY, "131072", 1048576.0)] * 3
    paths = [str(tmp_path / n) for n in ("sf.csv", "sw.csv", "cf.csv", "cw.csv")]
    write_counters(paths[0], fetch, "FETCH_SIZE")
    write_counters(paths[1], write, "WRITE_SIZE")
    write_counters(paths[2], cal_f, "FETCH_SIZE")
    write_counters(paths[3], cal_w, "WRITE_SIZE")
    out = io.StringIO()
    with redirect_stdout(out):
        bench.traffic_json(*paths, skip=2)
    d = json.loads(out.getvalue())
    # the first two dispatches of each pass are left out; the half-size ones
    # and the down launches never count
    assert d["dispatches"]["fetch"] == 5 and d["dispatches"]["write"] == 5
    assert d["copy_calibration"]["fetch_scale"] == 2.0 and d["copy_calibration"]["write_scale"] == 1.0
    assert d["hbm_fetch_bytes_per_launch"] == 23250 * 1024 * 2
    assert d["hbm_write_bytes_per_launch"] == 136 * 1024
    assert d["hbm_bytes_per_launch"] == 23250 * 2048 + 136 * 1024
    N, K = 34816, 5120
    assert d["algorithmic_bytes_per_launch"] == N * K // 4 + N * (K // 128) * 2 + 2 * K + 4 * N
    assert len(d["source_sha256_16"]) == 16


def test_trace_summary_runs(tmp_path):
    # 100 fused launches alone, a spin kernel, 95 alternating pairs of fused
    # and down, then a short run that is not reported
    rows = []
    t = 0

    def add(name, dur):
        nonlocal t
        rows.append({"Kernel_Name": name, "Grid_Size_X": "131072", "Start_Timestamp": t,
                     "End_Timestamp": t + dur})
        t += dur + 100

    for _ in range(100):
        add(FUSED, 10000)
    add("spin_kernel", 600000)
    for _ in range(95):
        add(FUSED, 11000)
        add(DOWN, 7000)
    for _ in range(5):
        add(DOWN, 7000)
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    out = io.StringIO()
    with redirect_stdout(out):
        bench.trace_summary(str(path))
    lines = out.getvalue().splitlines()[2:]
    assert len(lines) == 3, out.getvalue()
    first, alt_a, alt_b = ([c.strip() for c in l.split("|")] for l in lines)
    # averages leave out the first 10 dispatches of a run
    assert first[1] == "0" and first[3] == "100" and float(first[4]) == 10.0
    assert alt_a[1] == "101" and alt_a[3] == "95" and float(alt_a[4]) == 11.0
    assert alt_b[1] == "102 (alternating)" and alt_b[3] == "95" and float(alt_b[4]) == 7.0
    assert bench.TRAFFIC_KERNEL in first[2] and "64, 4, 8" in alt_b[2]
