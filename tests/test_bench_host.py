"""Host logic of the measurement tools (CPU only): the algorithmic byte count
of a step, the counter-traffic record and its source-hash gate, and the
per-block timeline summary."""
import csv
import importlib.util
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bench = _load("bench_under_test", os.path.join(ROOT, "bench.py"))
timeline = _load("timeline_under_test", os.path.join(ROOT, "gather_lora_matmul_amd", "timeline.py"))


def test_algorithmic_bytes_by_hand():
    # two slices, ranks 4 and 8, one adapter used twice, one id skipped
    wl = W.small_workload("bf16", 64, 96, [4, 8], 64, n_slices=2, seed=1)
    ids = np.array([0, 1, 0, -1], np.int32)
    want = 0
    for d_in, d_out in wl.slices:
        want += (4 + 8) * (d_in + d_out) * 2          # each distinct adapter once
        want += 4 * d_in * 2 + 2 * 4 * d_out * 2      # x once, y read + written
    assert bench.algorithmic_bytes(wl, ids, [0, 1], 2) == want
    # slices reading one x: x counted once
    shared = want - 4 * wl.slices[1][0] * 2
    assert bench.algorithmic_bytes(wl, ids, [0, 1], 2, shared_x=True) == shared
    # FP8 pages: one byte per code plus 2r fp32 scales per adapter slice
    wq = W.small_workload("e4m3", 64, 96, [4, 8], 64, n_slices=1, seed=1, act_dtype="f16")
    wantq = (4 + 8) * (64 + 96) * 1 + 8 * (4 + 8) + 4 * 64 * 2 + 2 * 4 * 96 * 2
    assert bench.algorithmic_bytes(wq, ids, [0], 2) == wantq


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, value in rows:
            w.writerow([name, counter, value])


def test_record_traffic_calibration_and_hash_gate(tmp_path):
    kern = "void lora::k_bgmv_apply<lora::f16_t, lora::f16_t, lora::f16_t, 512, 1, 2>(...)"
    copy = "__amd_rocclr_copyBuffer"
    mib64 = (64 << 20) / 1024
    # FETCH_SIZE reads half of the copy's 64 MiB; WRITE_SIZE all of it
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(copy, mib64 / 2)] * 10 + [(copy, 1.5)] * 3 +
                    [(kern, 1000.0), (kern, 3000.0), ("lora::k_scatter_pages(...)", 9e9)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(copy, mib64)] * 10 + [(kern, 100.0), (kern, 300.0)])
    out = tmp_path / "traffic.json"
    rec = bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "wl", "lora_bgmv_apply",
                               "abc", ["cmd"], path=str(out))
    assert abs(rec["fetch_factor"] - 2.0) < 1e-12 and abs(rec["write_factor"] - 1.0) < 1e-12
    # means over the step kernel's dispatches, set-up kernels excluded
    assert abs(rec["hbm_bytes_per_step"] - (2000.0 * 2 + 200.0) * 1024) < 1e-6
    tj = json.loads(out.read_text())
    assert tj["records"]["wl/lora_bgmv_apply"]["kernel_source_hash"] == "abc"
    got = bench.measured_traffic("wl", "lora_bgmv_apply", "abc", path=str(out))
    assert abs(got - rec["hbm_bytes_per_step"]) < 1e-6
    assert bench.measured_traffic("wl", "lora_bgmv_apply", "other", path=str(out)) is None
    assert bench.measured_traffic("wl", "lora_apply", "abc", path=str(out)) is None


def _rec(t0, t1, cu, slice_=0, rank=16, tok=0):
    # 100 MHz clock ticks; hardware id with the CU field at bits 11:8
    return [t0 * 100, t1 * 100, cu << 8, slice_, rank, tok, 0, 1]


def test_timeline_summary_serial_and_overlapping_blocks():
    # compute units are keyed by (block index % 8, wave id fields): blocks 0
    # and 8 run back to back on one unit with a 2 us gap; blocks 2 and 10 run
    # at once on another; the rest run alone
    recs = np.zeros((16, 8), np.uint64)
    recs[0] = _rec(0, 10, 0)
    recs[8] = _rec(12, 20, 0)
    for i in range(1, 8):
        recs[i] = _rec(0, 20, 0)
    recs[9] = _rec(0, 20, 1)
    recs[10] = _rec(5, 15, 0)        # same unit as block 2, inside its interval
    text = timeline.summarize(recs, "synthetic")
    assert "blocks 11, span 20.0 us" in text
    assert "at most 2 at once" in text
    # the only idle gap is the 2 us between blocks 0 and 8
    assert "median 2.00 us, p90 2.00, max 2.00" in text
