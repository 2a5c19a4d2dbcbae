"""bench.py's summaries of rocprofv3 output (host only): the timed-dispatch
selection of the kernel-trace table, the per-dispatch counter means, and the
copy-calibrated HBM byte record.  Synthetic CSV files in rocprofv3's column
layout stand in for a profiled run."""
import csv
import json
import os

import pytest

import bench

STEP = "void ra::(anonymous namespace)::attn_step_bf16_kernel<128, false>(ra::StepParams)"


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_short_kernel_names():
    assert bench._short_kernel(STEP) == "attn_step_bf16_kernel<128, false>"
    assert bench._short_kernel("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    long = ("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<bool, at::native::func_wrapper_t<bool, "
            "at::native::and_kernel_cuda(at::TensorIterator&)::{lambda()#1}> > >(at::native::ReduceOp<bool>)")
    assert bench._short_kernel(long).startswith("at::native::reduce_kernel<512, 1,")
    assert not bench._short_kernel(long).endswith(")")
    vec = ("void ra::(anonymous namespace)::relayout_kernel<unsigned int __vector(4)>(int, unsigned int, "
           "unsigned int __vector(4) const*, unsigned int __vector(4)*)")
    assert bench._short_kernel(vec) == "relayout_kernel<unsigned int __vector(4)>"


def test_trace_summary_takes_only_timed_dispatches(tmp_path):
    # 2 launches per ring step; warmup 1, steps 2: dispatches are
    # [w w | t t t t | w' w' | l l l l]; durations mark each group
    warmup, steps, n = 1, 2, 2
    durs = [9.0] * (warmup * n) + [2.0] * (steps * n) + [9.0] * n + [3.0] * (steps * n)
    rows, t = [], 1000
    for i, d in enumerate(durs):
        rows.append({"Dispatch_Id": i + 1, "Kernel_Name": STEP, "Start_Timestamp": t,
                     "End_Timestamp": t + int(d * 1000)})
        t += 100000
    rows.append({"Dispatch_Id": 99, "Kernel_Name": "__amd_rocclr_copyBuffer", "Start_Timestamp": 0,
                 "End_Timestamp": 500})
    rows.append({"Dispatch_Id": 100, "Kernel_Name": "void lib::k<" + "x" * 300 + ">", "Start_Timestamp": 0,
                 "End_Timestamp": 400})
    _write(str(tmp_path / "kt" / "kt_kernel_trace.csv"), rows,
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
    out = bench.trace_summary(str(tmp_path / "kt"), warmup, steps)
    assert "| `attn_step_bf16_kernel<128, false>` | 12 |" in out
    assert "| `lib::k<" + "x" * 90 + "...` | 1 |" in out   # long names cut to 100 characters
    assert "timed ring steps: 4 dispatches, mean 2.0 us" in out
    assert "timed per-launch repetitions: 4 dispatches, mean 3.0 us" in out
    assert "2 launches per ring step" in out


def _counter_rows(kernel, counter, values, instances=1):
    rows = []
    for i, v in enumerate(values):
        for k in range(instances):
            rows.append({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter,
                         "Counter_Value": v / instances})
    return rows


def test_counter_means_sum_instances_then_average(tmp_path):
    rows = _counter_rows(STEP, "SQ_INSTS_MFMA", [10.0, 30.0], instances=4)
    rows += _counter_rows("other_kernel(int)", "SQ_INSTS_MFMA", [1e9])
    _write(str(tmp_path / "c" / "c_counter_collection.csv"), rows,
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
    m = bench.counter_means([str(tmp_path / "c")])
    assert m["SQ_INSTS_MFMA"] == (pytest.approx(20.0), 2)


def test_traffic_record_scales_by_the_copy(tmp_path, monkeypatch):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(str(tmp_path / "f" / "c_counter_collection.csv"), _counter_rows(STEP, "FETCH_SIZE", [1000.0, 1000.0]),
           fields)
    _write(str(tmp_path / "w" / "c_counter_collection.csv"), _counter_rows(STEP, "WRITE_SIZE", [2048.0]), fields)
    # the copy of 1 GiB reads as 512 MiB on FETCH_SIZE and 1 GiB on WRITE_SIZE
    copy = "void at::native::copy_kernel(int)"
    _write(str(tmp_path / "cf" / "c_counter_collection.csv"),
           _counter_rows(copy, "FETCH_SIZE", [524288.0] * 3) + _counter_rows("fill(int)", "FETCH_SIZE", [0.0]), fields)
    _write(str(tmp_path / "cw" / "c_counter_collection.csv"),
           _counter_rows(copy, "WRITE_SIZE", [1048576.0] * 3), fields)
    rec = bench.traffic_summary(*(str(tmp_path / d) for d in ("f", "w", "cf", "cw")), "wl", ["cmd"])
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == 2 * 1000 * 1024
    assert rec["write_bytes_per_launch"] == 2048 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["kernel_hash"] == bench.kernel_hash()
    json.dumps(rec)


def test_measured_traffic_requires_the_current_kernel(tmp_path, monkeypatch):
    f = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({"workload": "wl", "kernel_hash": "stale", "bytes_per_launch": 5}))
    assert bench.measured_traffic("wl") is None
    f.write_text(json.dumps({"workload": "wl", "kernel_hash": bench.kernel_hash(), "bytes_per_launch": 5}))
    assert bench.measured_traffic("wl") == 5
    assert bench.measured_traffic("other") is None
