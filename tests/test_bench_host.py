"""Host-side logic of bench.py that needs no GPU: the one-GPU guard and the
counter-traffic summary (calibration against a plain copy of known size)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(path, counter, copy_kib, kern_rows):
    names = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
             "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
             "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
             "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=names)
        wr.writeheader()
        rows = [("__amd_rocclr_copyBuffer", copy_kib)] * 3 + [("__amd_rocclr_copyBuffer", 0.5)]
        rows += kern_rows
        for i, (name, v) in enumerate(rows):
            wr.writerow({**{k: 0 for k in names}, "Dispatch_Id": i, "Kernel_Name": name,
                         "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    import bench
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    k1 = "void lora::(anonymous namespace)::shrink_kernel<unsigned short, 3, 1>(lora::ShrinkArgs)"
    k2 = "lora::(anonymous namespace)::reduce_slabs(float const*, long, int, float*, long)"
    f = tmp_path / "fetch.csv"
    w = tmp_path / "write.csv"
    # copy of 256 MiB: FETCH reads half (128 MiB), WRITE reads all
    _write_counters(f, "FETCH_SIZE", 131072.0, [(k1, 1000.0), (k1, 1000.0), (k2, 10.0), (k2, 10.0)])
    _write_counters(w, "WRITE_SIZE", 262144.0, [(k1, 20.0), (k1, 20.0), (k2, 5.0), (k2, 5.0)])
    args = type("A", (), {"traffic_from": [str(f), str(w)], "traffic_kind": "shrink_qkv",
                          "workload": "prefill"})()
    bench.summarize_traffic(args)
    out = json.load(open(tmp_path / "traffic.json"))
    assert out["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert out["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    # per call: (1000 + 10) KiB fetched x 2 + (20 + 5) KiB written
    want = (1010.0 * 2 + 25.0) * 1024
    assert out["kernels"]["prefill:shrink_qkv"]["hbm_bytes_per_launch"] == pytest.approx(want)


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """The hash that ties profiles/traffic.json to a kernel source changes with
    the code and with string literals, not with comments or blank lines."""
    import bench
    base = ('// header\n#include <x.h>\n/* block\n   comment */\nint f(int a) { return a + 1; }  // tail\n'
            'const char* s = "not // a comment";\n')
    variants = {
        "base": base,
        "comments": base.replace("// header", "// another header\n\n").replace("// tail", "/* t */"),
        "code": base.replace("a + 1", "a + 2"),
        "string": base.replace("not // a comment", "not // a remark"),
    }
    h = {}
    for k, src in variants.items():
        p = tmp_path / f"{k}.hip"
        p.write_text(src)
        monkeypatch.setattr(bench, "KERNEL_SRC", str(p))
        h[k] = bench.kernel_sha()
    assert h["comments"] == h["base"]
    assert h["code"] != h["base"]
    assert h["string"] != h["base"]


def test_trace_summary_attributes_dispatches_to_timing_ranges(tmp_path, capsys):
    """Two call kinds that share a kernel and a grid are told apart by the
    per-call timing ranges of the marker trace; dispatches outside every
    range (the timed steps) and ranges without a 'workload:kind' name are
    not attributed."""
    import bench
    name = "void lora::(anonymous namespace)::fused_delta_kernel<1, 8, true, true, false, 0>(lora::FusedArgs)"
    with open(tmp_path / "p_kernel_stats.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writerow([name, 5, 35000, 7000, 100.0, 6000, 8000, 0])
    cols = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Workgroup_Size_Y",
            "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    rows = [(100, 108), (1000, 1007), (1010, 1017), (2000, 2006), (2010, 2016)]
    with open(tmp_path / "p_kernel_trace.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(cols)
        for a, b in rows:
            wr.writerow(["KERNEL_DISPATCH", name, a * 1000, b * 1000, 1024, 1, 1, 1024 * 128, 2, 1])
    with open(tmp_path / "p_marker_api_trace.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Domain", "Function", "Process_Id", "Thread_Id", "Correlation_Id", "Start_Timestamp",
                     "End_Timestamp"])
        wr.writerow(["MARKER_CORE_RANGE_API", "decode:delta_qkv", 1, 1, 1, 990 * 1000, 1020 * 1000])
        wr.writerow(["MARKER_CORE_RANGE_API", "decode:delta_o", 1, 1, 2, 1990 * 1000, 2020 * 1000])
        wr.writerow(["MARKER_CORE_RANGE_API", "unrelated", 1, 1, 3, 0, 3000 * 1000])
    bench.trace_summary(str(tmp_path / "p_kernel_stats.csv"), str(tmp_path / "p_kernel_trace.csv"))
    out = capsys.readouterr().out
    kinds = [ln.split() for ln in out.split("(workload:call kind):")[1].splitlines() if ln.startswith("decode:")]
    assert [(k[0], k[-3], k[-2]) for k in kinds] == [("decode:delta_o", "2", "6.00"), ("decode:delta_qkv", "2", "7.00")]
