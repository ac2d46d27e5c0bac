"""Host-side logic of bench.py (no GPU): the multi-GPU refusal and the
counter record that feeds the roofline's `traffic` field."""
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


def test_traffic_record_belongs_to_its_workload_and_recipe():
    # The committed records cover the 1000-view workload only; another
    # workload or a recipe without a record gets no traffic figure.
    assert bench.load_traffic("mse_gd", "views2000") is None
    assert bench.load_traffic("dot_gd", "views1000") is None
    for recipe in ("mse_gd", "dot_muon"):
        t = bench.load_traffic(recipe, "views1000")
        # None only if the gradient kernel's source changed since the counters were taken
        assert t is None or 5.0e9 < t < 6.5e9
