"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic
FLOP and byte counts it reports, and the summarisers that turn rocprofv3 output
into the files under profiles/ (fed here with small synthetic counter files).
"""

import csv
import json
import os
import sqlite3
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402

# Attention GFLOP of rank 0's problem (4 B H Sq Skv D) and pack bytes (Q, K and V of
# the local shard read once and written once) for the four unmasked workloads, worked
# out by hand from their shapes, e.g. video: 4 x 6 x 16380 x 32760 x 128 flops and
# 2 x 3 x 8190 x 12 x 128 x 2 bytes.
TABLE = {
    "tiny_w2": (0.0336, 393_216),
    "image_cp4": (58.18, 40_108_032),
    "image_cp8": (25.77, 18_874_368),
    "video_u2a2": (1648.46, 150_958_080),
}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


@pytest.mark.parametrize("name", sorted(TABLE))
def test_flops_and_bytes_match_the_configurations(name):
    wl = workloads.WORKLOADS[name]
    gflop, pack = TABLE[name]
    assert wl.pack_bytes() == pack
    assert round(bench.attn_flops(wl, workloads.key_mask(wl)) / 1e9, 2 if gflop > 1 else 4) == gflop


def test_masked_flops_count_only_valid_keys():
    wl = workloads.WORKLOADS["joint_cfg_cp4"]
    mask = workloads.key_mask(wl)
    valid = mask.astype(np.int64).sum(axis=1)
    # image keys always valid, then a text prefix of 64..512 tokens per batch row
    assert ((valid >= 4096 + 64) & (valid <= 4096 + 512)).all()
    assert bench.attn_flops(wl, mask) == 4 * wl.attn_heads * wl.attn_rows * wl.D * int(valid.sum())
    assert bench.attn_flops(wl, None) == wl.attn_flops_dense() == 4 * 2 * 24 * 1152 * 4608 * 128


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for kernel, counter, value in rows:
            w.writerow([kernel, counter, value])


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    kib = bench.CALIB_BYTES / 1024.0
    # the copy's counters read 2x (fetch) and 0.5x (write) its true bytes
    _counter_csv(os.path.join(fetch, "copy"), [("copyBuffer", "FETCH_SIZE", 2 * kib)])
    _counter_csv(os.path.join(write, "copy"), [("copyBuffer", "WRITE_SIZE", 0.5 * kib)])
    _counter_csv(os.path.join(fetch, "attn"), [("attn_fwd_kernel<128, 0>", "FETCH_SIZE", 1000.0),
                                               ("attn_fwd_kernel<128, 0>", "FETCH_SIZE", 3000.0)])
    _counter_csv(os.path.join(write, "attn"), [("attn_fwd_kernel<128, 0>", "WRITE_SIZE", 500.0)])
    out = str(tmp_path / "traffic.json")
    bench.summarize_traffic(fetch, write, out, "image_cp4")
    res = json.load(open(out))
    assert res["scale_fetch"] == pytest.approx(0.5) and res["scale_write"] == pytest.approx(2.0)
    assert res["traffic_bytes"] == pytest.approx((2000.0 * 0.5 + 500.0 * 2.0) * 1024.0)
    assert res["src_sha256"] == bench.src_sha256()


def test_trace_summary_reports_the_attention_kernel(tmp_path):
    db = str(tmp_path / "kt.db")
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
                "percentage real)")
    con.executemany("insert into top_kernels values (?, ?, ?, ?, ?)", [
        ("void cpattn::(anonymous namespace)::attn_fwd_kernel<128, 0>(cpattn::AttnArgs)", 10, 600.0, 60.0, 90.0),
        ("void cpattn::(anonymous namespace)::permute_kernel<PackMap<16>, true>(PackMap<16>)", 10, 50.0, 5.0, 10.0),
    ])
    con.commit()
    con.close()
    out = str(tmp_path / "kt.md")
    bench.summarize_trace(db, out, "rocprofv3 --kernel-trace --stats -- python3 bench.py", "image_cp4")
    text = open(out).read()
    assert "| `attn_fwd_kernel<128, 0>` | 10 | 600.0 | 60.000 | 90.00% |" in text
    flops = workloads.WORKLOADS["image_cp4"].attn_flops_dense()
    tf = flops / 60e-6 / 1e12
    assert f"{tf:.1f} TFLOP/s = {100.0 * tf / 2500.0:.1f}% of the 2.5 PFLOP/s" in text


def test_trace_summary_sums_the_launches_of_one_call(tmp_path):
    # a call that runs its heads in two launches (256-row and 128-row blocks)
    db = str(tmp_path / "kt2.db")
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
                "percentage real)")
    con.executemany("insert into top_kernels values (?, ?, ?, ?, ?)", [
        ("void cpattn::(anonymous namespace)::attn_fwd_kernel<128, 64>(cpattn::AttnArgs)", 4, 3600.0, 900.0, 60.0),
        ("void cpattn::(anonymous namespace)::attn_fwd_kernel<128, 0>(cpattn::AttnArgs)", 4, 1800.0, 450.0, 30.0),
    ])
    con.commit()
    con.close()
    out = str(tmp_path / "kt2.md")
    bench.summarize_trace(db, out, "cmd", "video_u2a2")
    text = open(out).read()
    tf = workloads.WORKLOADS["video_u2a2"].attn_flops_dense() / 1350e-6 / 1e12
    assert "/ 1350.00 us" in text and f"{tf:.1f} TFLOP/s" in text


def test_traffic_sums_the_launches_of_one_call(tmp_path):
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    kib = bench.CALIB_BYTES / 1024.0
    _counter_csv(os.path.join(fetch, "copy"), [("copyBuffer", "FETCH_SIZE", kib)])
    _counter_csv(os.path.join(write, "copy"), [("copyBuffer", "WRITE_SIZE", kib)])
    _counter_csv(os.path.join(fetch, "attn"), [("attn_fwd_kernel<128, 64>", "FETCH_SIZE", 300.0),
                                               ("attn_fwd_kernel<128, 0>", "FETCH_SIZE", 100.0),
                                               ("attn_fwd_kernel<128, 64>", "FETCH_SIZE", 500.0),
                                               ("attn_fwd_kernel<128, 0>", "FETCH_SIZE", 100.0)])
    _counter_csv(os.path.join(write, "attn"), [("attn_fwd_kernel<128, 64>", "WRITE_SIZE", 10.0),
                                               ("attn_fwd_kernel<128, 0>", "WRITE_SIZE", 20.0)])
    out = str(tmp_path / "traffic2.json")
    bench.summarize_traffic(fetch, write, out, "video_u2a2")
    res = json.load(open(out))
    assert res["traffic_bytes"] == pytest.approx((400.0 + 100.0 + 30.0) * 1024.0)
