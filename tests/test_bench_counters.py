"""bench.py's counter summary on synthetic rocprofv3 output (no GPU): the
dispatches are attributed to the manifest in launch order, launches of other
kernels in between are skipped, and the bytes are calibrated by the copy."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, dispatches, counter, values):
    os.makedirs(path)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(zip(dispatches, values)):
            w.writerow({"Correlation_Id": i + 1, "Dispatch_Id": i + 1, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": 1024, "Kernel_Id": 1, "Kernel_Name": name,
                        "Workgroup_Size": 256, "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 8,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 16, "Counter_Name": counter, "Counter_Value": v,
                        "Start_Timestamp": 0, "End_Timestamp": 1})


def test_summary_attribution_and_calibration(tmp_path, capsys):
    calls = bench.COUNTER_CALLS
    entries = [
        {"label": "a fwd", "kernel": "rmsnorm_fwd_kernel", "calls": calls, "algorithmic_bytes": 4 << 20,
         "scratch_bytes": 0, "workload": "w"},
        {"label": "a bwd_rows", "kernel": "rmsnorm_bwd_rows_kernel", "calls": calls, "algorithmic_bytes": 6 << 20,
         "scratch_bytes": 1 << 20, "workload": "w"},
        {"label": "copy", "kernel": bench.COPY_KERNEL, "calls": calls, "algorithmic_bytes": 2 * bench.COPY_BYTES,
         "scratch_bytes": 0, "workload": "copy"},
    ]
    json.dump({"kernel_sha": "0123456789abcdef", "entries": entries}, open(tmp_path / "manifest.json", "w"))
    # a set-up launch of the backward before the forwards, an unrelated fill
    # kernel before the copies; the copy's FETCH_SIZE reads half its bytes
    names = (["rmsnorm_bwd_rows_kernel"] + ["rmsnorm_fwd_kernel"] * calls + ["rmsnorm_bwd_rows_kernel"] * calls
             + ["fill_kernel"] + [f"void at::native::{bench.COPY_KERNEL}<...>"] * calls)
    half_kib = bench.COPY_BYTES / 1024 / 2
    fetch = [9e9] + [1024.0] * calls + [2048.0, 2048.0, 4096.0] + [5.0] + [half_kib] * calls
    write = [9e9] + [2048.0] * calls + [1024.0] * calls + [5.0] + [2 * half_kib] * calls
    _write(str(tmp_path / "fetch"), names, "FETCH_SIZE", fetch)
    _write(str(tmp_path / "write"), names, "WRITE_SIZE", write)
    bench.summarize_counters(str(tmp_path))
    out = capsys.readouterr().out
    data = json.loads(out.split("```json\n")[1].split("\n```")[0])
    assert data["fetch_scale"] == pytest.approx(2.0) and data["write_scale"] == pytest.approx(1.0)
    e = data["entries"]
    # forward: 1024 KiB fetched (x2), 2048 KiB written: 4 MiB moved = its algorithmic bytes
    assert e["a fwd"]["scaled_bytes"] == 4 << 20 and e["a fwd"]["ratio"] == pytest.approx(1.0)
    # backward: the median of its three launches (not the set-up launch)
    assert e["a bwd_rows"]["fetch_kib"] == 2048.0
    assert e["a bwd_rows"]["scaled_bytes"] == (2 * 2048 + 1024) * 1024
    assert e["copy"]["scaled_bytes"] == 2 * bench.COPY_BYTES


def test_traffic_table_requires_matching_sources(tmp_path, monkeypatch):
    summary = tmp_path / "s.md"
    summary.write_text("text\n```json\n" + json.dumps({"kernel_sha": "abc", "entries": {
        "rms c3 bwd_rows": {"scaled_bytes": 123}}}) + "\n```\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    assert bench.traffic_table("abc") == {"rms c3 bwd_rows": 123}
    assert bench.traffic_table("other") == {}
