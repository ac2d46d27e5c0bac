"""Host-side logic of bench.py (no GPU): the multi-GPU refusal and the
counter record that feeds the roofline's `traffic` and clock fields."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_counter_record_belongs_to_its_workload_recipe_and_kernel():
    # Records exist for the 1000-view workload (both recipes) and the 2000-view
    # one (squared error); another recipe, or another gradient kernel than the
    # one the record was taken on, gets none.
    pipe, dot = bench.GRAD_KERNEL["mse"], bench.GRAD_KERNEL["dot"]
    assert bench.load_counter_record("dot_gd", "views1000", dot) is None
    assert bench.load_counter_record("mse_gd", "views1000", "grad_partial_bf16_kernel (with loss value)") is None
    assert bench.load_counter_record("mse_gd", "views1000", dot) is None
    for recipe, cfg, kernel, n in (("mse_gd", "views1000", pipe, 1374000), ("dot_muon", "views1000", dot, 1374000),
                                   ("mse_gd", "views2000", pipe, 2748000)):
        rec = bench.load_counter_record(recipe, cfg, kernel)
        # None only if the gradient kernel's source changed since the counters were taken
        if rec is None:
            continue
        algorithmic = n * 4096  # K and V' rows of 16 heads x 64 bf16
        assert algorithmic < rec["traffic_bytes_per_launch"] < 1.05 * algorithmic
        # a shader clock between idle-ish and the 2.4 GHz peak, consistent with its own figures
        assert 1.0 < rec["clock_GHz"] <= bench.SPEC_CLOCK_GHZ
        assert abs(rec["clock_GHz"] - rec["gpu_active_cycles_per_xcd"] / rec["event_timed_launch_ms"] / 1e6) < 1e-3
