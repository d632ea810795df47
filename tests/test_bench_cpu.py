"""The measurement code of bench.py, on the CPU: byte and flop counts, the
rocprofv3 ingest (on synthetic CSV files of the shape rocprofv3 writes) and
the one-GPU refusal.  Nothing here touches a GPU or the committed profiles."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_counts_follow_the_shapes():
    b, h, s, d, n, p = bench.ATTN
    assert bench._attn_flops() == 2 * 2 * b * h * s * n * d          # q k^T and P v
    qkv = b * h * s * d * 2 + 2 * b * h * n * d * 2                   # bf16 reads
    assert bench._attn_bytes() == qkv + p * b * h * s * (d + 2) * 4   # O, m, l float32
    assert bench._attn_fused_bytes() == qkv + b * h * s * d * 2       # bf16 out
    assert bench.NEXT_BYTES["attention_fused"] == bench.NEXT_BYTES["attention_merged"]


def test_every_timed_kernel_has_algorithmic_bytes():
    algo = bench._algo_bytes()
    assert set(bench.KERNEL_OF_OP) <= set(algo)
    assert all(v > 0 for v in algo.values())
    # the step's ops move what the docstring says: e.g. the long rows read
    # 16 x 2^24 floats and write 16
    assert algo["long_sum"] == 16 * (1 << 24) * 4 + 16 * 4


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_counter_ingest_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "prof" / "traffic.json"))
    sym = bench.KERNEL_OF_OP["long_sum"]
    copy = "void at::native::neg_kernel_impl(float)"
    # three dispatches of 150, 151 and 155 us, and the reference read at its
    # two sizes: 1 GiB in 150 us and 128 MiB in 21 us
    disp = [("void rr::%s(float const*)" % sym, 150000), ("void rr::%s(float const*)" % sym, 151000),
            ("void rr::%s(float const*)" % sym, 155000), ("void rr::k_stream<0>(x)", 150000),
            ("void rr::k_stream<0>(x)", 21000)]
    _write_csv(str(tmp_path / "trace" / "x" / "t_kernel_trace.csv"),
               [{"Kernel_Name": n, "Start_Timestamp": str(1000 * i),
                 "End_Timestamp": str(1000 * i + d)} for i, (n, d) in enumerate(disp)])
    half = bench.COPY_BYTES / 1024.0 / 2   # FETCH_SIZE reads half the bytes on this part
    for d, name, k_val, c_val in (("fetch", "FETCH_SIZE", 524288.0, half),
                                  ("write", "WRITE_SIZE", 0.0625, bench.COPY_BYTES / 1024.0)):
        _write_csv(str(tmp_path / d / "y" / "c_counter_collection.csv"),
                   [{"Kernel_Name": "void rr::%s(float const*)" % sym, "Counter_Name": name,
                     "Counter_Value": str(k_val)},
                    {"Kernel_Name": copy, "Counter_Name": name, "Counter_Value": str(c_val)}])
    out, table = bench.ingest_counters(str(tmp_path / "trace"), str(tmp_path / "fetch"),
                                       str(tmp_path / "write"))
    k = out["kernels"]["long_sum"]
    assert out["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert out["calibration"]["write_scale"] == pytest.approx(1.0)
    assert k["fetch_bytes"] == 1 << 30 and k["write_bytes"] == 64
    assert k["traffic_over_algorithmic"] == pytest.approx(1.0, abs=1e-3)
    assert out["source_hash"] == bench.kernel_source_hash()
    assert "| 3 | 152.0 | 151.0 | 150.0 | 155.0 |" in table
    # one kernel at two sizes: each op keeps its own dispatch
    assert "(stream_read) | 1 | 150.0 |" in table
    assert "(stream_read_128MiB) | 1 | 21.0 |" in table
    assert json.load(open(bench.TRAFFIC_FILE))["kernels"]["long_sum"]["bytes_per_launch"] == (1 << 30) + 64


def test_sq_summary_averages_the_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "prof" / "traffic.json"))
    os.makedirs(str(tmp_path / "prof"))
    sym = bench.KERNEL_OF_OP["attention"]
    rows = [{"Kernel_Name": "void rr::%s(...)" % sym, "Counter_Name": "SQ_INSTS_MFMA",
             "Counter_Value": v} for v in ("4", "6")]
    rows.append({"Kernel_Name": "other", "Counter_Name": "SQ_INSTS_MFMA", "Counter_Value": "100"})
    _write_csv(str(tmp_path / "sq0" / "s_counter_collection.csv"), rows)
    path = bench.sq_summary("attention", [str(tmp_path / "sq0")])
    text = open(path).read()
    assert "| SQ_INSTS_MFMA | 5 | 2 |" in text
    assert "--only attention" in text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0 and "one GPU only" in r.stderr
