"""CPU checks of bench.py's contract: the metric formulas against the
per-configuration figures worked out by hand from the shapes (sketch FLOPs
2 T r (d + k) per matrix and microbatch; apply bytes W read and written, S
once, v, v'), and the refusal of more than one GPU (no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rank_gradient_sketching_sketch_amd import inputs  # noqa: E402

# (workload, sketch FLOP per step, apply bytes per step), from the shapes:
# e.g. the 7B up projection: 2 * 4096 * 256 * (18944 + 3584) * 16 microbatches
# = 755.9 GFLOP; its apply 2 * 2 * 18944 * 3584 + 4 * 18944 * 256 + 12 * 18944
# = 291.2 MB.
HAND_FIGURES = [
    ("tiny_fp32", 25.17e6, 1.084e6),
    ("qwen1.5b_set", 345.7e9, 211.0e6),
    ("qwen7b_up", 755.9e9, 291.2e6),
    ("qwen7b_28layer", 42.33e12, 27.54e9),
    ("27b_64layer", 215.5e12, 88.02e9),
]


@pytest.mark.parametrize("name,flop,apply_bytes", HAND_FIGURES)
def test_metric_formulas_match_hand_figures(name, flop, apply_bytes):
    wl = inputs.WORKLOADS[name]
    assert bench.sketch_flop_per_step(wl) == pytest.approx(flop, rel=1e-3)
    assert bench.apply_bytes_per_step(wl) == pytest.approx(apply_bytes, rel=1e-3)


def test_fold_bytes_of_the_headline_launch():
    # dY 2Td + P 2Tr + S 4dr written, plus S read on 15 of 16 launches
    wl = inputs.WORKLOADS["qwen7b_up"]
    T, d, r = 4096, 18944, 256
    per_step = 16 * (2 * T * d + 2 * T * r + 4 * d * r) + 15 * 4 * d * r
    assert bench.fold_bytes_per_step(wl) == per_step
    assert per_step // 16 == 194871296


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_fold_bytes_per_launch():
    T, d, r = 4096, 18944, 256
    assert bench.fold_bytes_per_launch(T, d, r, True) == 196083712
    assert bench.fold_bytes_per_launch(T, d, r, False) == 196083712 - 4 * d * r


def test_traffic_record_is_tied_to_the_fold_sources(monkeypatch):
    rec = bench.fold_traffic_record("qwen7b_up")
    # the committed record parses and carries counter bytes per dispatch
    # (None only if the fold sources changed after the counters were taken)
    if rec is not None:
        assert rec["fold_bytes_per_dispatch"] > bench.fold_bytes_per_launch(4096, 18944, 256, True)
        assert rec["fold_sources_sha256"] == bench.fold_sources_sha256()
    rec_fold = bench.fold_traffic_record("qwen7b_up", "logra_sketch_fold")
    if rec_fold is not None:
        assert rec_fold["fold_bytes_per_dispatch"] > bench.fold_bytes_per_launch(4096, 18944, 256, True)
    assert bench.fold_traffic_record("qwen7b_up", "no_such_call") is None
    monkeypatch.setattr(bench, "fold_sources_sha256", lambda: "0" * 64)
    assert bench.fold_traffic_record("qwen7b_up") is None
    assert bench.fold_traffic_record("qwen7b_up", "logra_sketch_fold") is None
    assert bench.fold_traffic_record("no_such_workload") is None
