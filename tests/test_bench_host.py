"""Host-side checks of bench.py's contract (no GPU): one GPU only, and the
CPU baseline object for every workload mode."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from w8a8_quantized_linear_sq_amd import inputs  # noqa: E402


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env={**os.environ, **(env or {})}, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_multi_rank_launch_is_refused():
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert r.stdout == ""


@pytest.mark.parametrize("mode", ["full", "per_call", "per_tensor", "weight_only"])
def test_cpu_baseline_object(mode):
    case = inputs.tiny()
    cb = bench.cpu_baseline(case, mode, 0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TOPS"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["sample"], str) and cb["sample"]
    assert cb["seconds_measured"] >= 0
    if mode == "full":
        # the tiny layer fits the budget: whole steps repeated until it is spent
        assert "whole steps" in cb["sample"] and cb["seconds_measured"] >= 0.2 or "50 whole steps" in cb["sample"]


def test_every_workload_names_a_case_and_mode():
    for name, (desc, spec, mode) in bench.WORKLOADS.items():
        assert desc and mode in ("full", "per_call", "per_tensor", "weight_only"), name
        assert hasattr(inputs, spec[0]), name
