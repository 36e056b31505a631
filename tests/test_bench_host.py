"""Host-side checks of bench.py: the one-GPU guard and the counter-summary round trip
(synthetic rocprofv3 CSVs; no GPU)."""
import argparse
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from weight_merge_amd.configs import PRESETS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def _csv(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_round_trip(tmp_path):
    merge = "void ada::(anonymous namespace)::merge_bf16_kernel<32, 2, 4, 2, 0, false>(ada::MergeParams)"
    neg = "void at::native::vectorized_elementwise_kernel<8, at::native::neg_kernel_cuda>(int)"
    other = "void at::native::fill_kernel(int)"
    d = {k: str(tmp_path / k) for k in ("f", "w", "cf", "cw")}
    # two merge dispatches (1000 and 1200 KiB fetched, 2000 written) and an unrelated kernel
    _csv(d["f"], [{"Dispatch_Id": 1, "Kernel_Name": merge, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000},
                  {"Dispatch_Id": 2, "Kernel_Name": merge, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1200},
                  {"Dispatch_Id": 3, "Kernel_Name": other, "Counter_Name": "FETCH_SIZE", "Counter_Value": 9e9}])
    _csv(d["w"], [{"Dispatch_Id": 1, "Kernel_Name": merge, "Counter_Name": "WRITE_SIZE", "Counter_Value": 2000}])
    # calibration over 1 MiB: the fetch counter reads half, the write counter all of it
    _csv(d["cf"], [{"Dispatch_Id": 5, "Kernel_Name": neg, "Counter_Name": "FETCH_SIZE", "Counter_Value": 512}])
    _csv(d["cw"], [{"Dispatch_Id": 5, "Kernel_Name": neg, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024}])
    args = argparse.Namespace(traffic_from=[d["f"], d["w"], d["cf"], d["cw"]], calibrate_mib=1, out_of_place=False)
    cfg = PRESETS["llama7b_e8r16k2"]
    out = str(tmp_path / "traffic.txt")
    bench.write_traffic(args, cfg, out)
    expect = 1100 * 1024 * 2.0 + 2000 * 1024 * 1.0
    assert bench.read_traffic(cfg.name, "in_place", out) == pytest.approx(expect)
    assert bench.read_traffic(cfg.name, "out_of_place", out) is None
    assert bench.read_traffic("llama7b_e16r64k4", "in_place", out) is None
    text = open(out).read().replace(bench.kernel_sha(), "0" * 16)
    open(out, "w").write(text)
    assert bench.read_traffic(cfg.name, "in_place", out) is None  # taken on another kernel source


def test_kernel_identity_ignores_comments():
    code = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    assert bench._code_only(code) == bench._code_only("/* doc\n   more */\n" + code.replace("// add one", "// +1"))
    assert bench._code_only(code) != bench._code_only(code.replace("+ 1", "+ 2"))


def test_trace_summary_separates_timed_from_warm_up_launches(tmp_path):
    """A synthetic rocprofv3 kernel trace of 1 warm-up and 2 timed steps: the summary
    averages the last 2 x steps merge launches (merge and unmerge alternate) apart from
    the warm-up ones."""
    merge = "void ada::(anonymous namespace)::merge_bf16_kernel<32, 1, 8, 2, 0, false, 1>(ada::MergeParams)"
    pre = "void ada::(anonymous namespace)::pregate_kernel<unsigned short>(...)"
    folder = tmp_path / "trace"
    folder.mkdir()
    rows, t = [], 0
    for dur in (9000, 9000, 4000, 4200, 4400, 4600):  # ns: warm-up merge+unmerge, then two timed steps
        rows.append({"Kernel_Name": pre, "Start_Timestamp": t, "End_Timestamp": t + 5000})
        t += 10000
        rows.append({"Kernel_Name": merge, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 100
    with open(folder / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)
    out = str(tmp_path / "summary.md")
    args = argparse.Namespace(trace_summary=[str(folder), out], steps=2, warmup=1, trace_command="rocprofv3 ...")
    bench.trace_summary(args, PRESETS["llama7b_e8r16k2"])
    text = open(out).read()
    assert "timed launches: mean 4.3 µs" in text
    assert "warm-up launches: mean 9.0 µs over 2" in text
    args.warmup = 2  # a count that does not match the trace is refused
    with pytest.raises(SystemExit):
        bench.trace_summary(args, PRESETS["llama7b_e8r16k2"])


def test_counter_summary_averages_per_dispatch(tmp_path):
    merge = "void ada::(anonymous namespace)::merge_bf16_kernel<64, 4, 4, 2, 3, true, 2>(ada::MergeParams)"
    d = str(tmp_path / "q1")
    # two dispatches, each counter reported per XCD (two rows summed per dispatch)
    _csv(d, [{"Dispatch_Id": 1, "Kernel_Name": merge, "Counter_Name": "SQ_WAVES", "Counter_Value": 10},
             {"Dispatch_Id": 1, "Kernel_Name": merge, "Counter_Name": "SQ_WAVES", "Counter_Value": 20},
             {"Dispatch_Id": 2, "Kernel_Name": merge, "Counter_Name": "SQ_WAVES", "Counter_Value": 50},
             {"Dispatch_Id": 3, "Kernel_Name": "other", "Counter_Name": "SQ_WAVES", "Counter_Value": 999}])
    out = str(tmp_path / "c.md")
    args = argparse.Namespace(counter_summary=[out, d], trace_command="rocprofv3 ...")
    bench.counter_summary(args, PRESETS["llama7b_e16r64k4"])
    assert "| SQ_WAVES | 40 | 2 | `q1` |" in open(out).read()
