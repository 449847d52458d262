"""Host-side logic of bench.py (CPU only): the single-GPU guard, the
algorithmic byte counts and the HBM counter summary."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from input_dependent_short_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


# Each input read once and each output written once, worked by hand per tensor
# (MB = 1e6 bytes; bf16 = 2 B, fp32 = 4 B; N = B*T tokens):
#   head-wise fwd: x + w + y;          bwd: x + w + dy + dx + dw
#   low-rank  fwd: x + z + U + y;      bwd: x + z + U + dy + dx + dz + dU (fp32)
BYTES = {
    # per-channel H = 1, fp32, N = 64, D = 64, W = 4: x, y 16384 B each, w 65536 B
    1: (16384 + 65536 + 16384, 3 * 16384 + 2 * 65536),
    # N = 16384, D = 2304, H = 64 (36 filters), W = 4: x 75.497472 MB, w 4.718592 MB
    2: (2 * 75.497472e6 + 4.718592e6, 3 * 75.497472e6 + 2 * 4.718592e6),
    # R = 32: z 1.048576 MB, U 0.589824 MB, dU 1.179648 MB
    3: (2 * 75.497472e6 + 1.048576e6 + 0.589824e6, 3 * 75.497472e6 + 2 * 1.048576e6 + 0.589824e6 + 1.179648e6),
    # N = 16384, D = 8192, H = 16 (512 filters): x 268.435456 MB, w 67.108864 MB
    4: (2 * 268.435456e6 + 67.108864e6, 3 * 268.435456e6 + 2 * 67.108864e6),
    # D = 6144, R = 64: x 201.326592 MB, z 2.097152 MB, U 3.145728 MB, dU 6.291456 MB
    5: (2 * 201.326592e6 + 2.097152e6 + 3.145728e6,
        3 * 201.326592e6 + 2 * 2.097152e6 + 3.145728e6 + 6.291456e6),
}


@pytest.mark.parametrize("cfg", sorted(BYTES))
def test_algorithmic_bytes(cfg):
    wl = inputs.WORKLOADS[cfg]
    es = 4 if wl.dtype == "fp32" else 2
    for direction, want in zip(("fwd", "bwd"), BYTES[cfg]):
        got = bench.algorithmic_bytes(wl.kind, direction, wl.B, wl.T, wl.D, wl.W, wl.H, wl.R, es=es)
        assert abs(got - want) < 1.0, f"cfg {cfg} {direction}: {got} vs {want}"


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_summary_scales_by_the_copy_and_adds_helper_launches(tmp_path):
    """The counters of a 1 GiB copy (1 GiB read, 1 GiB written) fix the scale
    of each counter; an entry point's bytes per call include the zero-fill and
    cast launches of the same call."""
    copy = "__amd_rocclr_copyBuffer"
    lrb = "void dsc::(anonymous namespace)::lr_bwd_mfma<4, 1, 4, true, 2>(dsc::LrParams, long, long)"
    fetch = [(copy, "FETCH_SIZE", 524288.0), (copy, "FETCH_SIZE", 100.0),   # reads half of 1 GiB; a small copy
             (lrb, "FETCH_SIZE", 1000.0), (lrb, "FETCH_SIZE", 1000.0),
             ("clear2(unsigned int*, long, unsigned int*, long)", "FETCH_SIZE", 10.0),
             ("clear2(unsigned int*, long, unsigned int*, long)", "FETCH_SIZE", 10.0),
             ("cast_f32_bf16", "FETCH_SIZE", 30.0), ("cast_f32_bf16", "FETCH_SIZE", 30.0)]
    write = [(copy, "WRITE_SIZE", 1048576.0), (lrb, "WRITE_SIZE", 500.0), (lrb, "WRITE_SIZE", 500.0)]
    _write_counters(str(tmp_path / "f"), fetch)
    _write_counters(str(tmp_path / "w"), write)
    out = str(tmp_path / "traffic.json")
    rec = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), out)
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    e = rec["entries"]["dsc_lowrank_bwd"]
    assert e["launches"] == 2
    assert e["fetch_bytes_per_launch"] == pytest.approx((1000 + 10 + 30) * 1024 * 2.0)
    assert e["write_bytes_per_launch"] == pytest.approx(500 * 1024 * 1.0)
    assert json.load(open(out))["kernel_source_hash"] == bench.kernel_source_hash()
