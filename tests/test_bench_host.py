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


def test_cpu_baseline_ste_object():
    case = inputs.tiny()
    dy = inputs.upstream_grad(case.m, case.n, seed=3, dtype="f32")
    cb = bench.cpu_baseline_ste(case, dy, 0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert f"of {case.m} tokens" in cb["sample"]
    assert cb["seconds_measured"] >= 0


def test_upstream_grad_is_seeded_and_bf16_exact():
    a = inputs.upstream_grad(5, 7, seed=11)
    b = inputs.upstream_grad(5, 7, seed=11)
    assert a.shape == (5, 7) and a.bits is not None
    assert (a.bits == b.bits).all()
    assert (inputs.bf16_to_f32(a.bits) == a.f32).all()


def test_every_workload_names_a_case_and_mode():
    for name, (desc, spec, mode) in bench.WORKLOADS.items():
        assert desc and mode in ("full", "per_call", "per_tensor", "weight_only", "ste"), name
        assert hasattr(inputs, spec[0]), name


def test_sclk_reading(tmp_path):
    """The amdgpu current-clock file (pp_dpm_sclk): the line marked '*' gives the clock
    (deep sleep and numbered levels alike); missing or unmarked: None."""
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 96Mhz\n0: 500Mhz\n1: 1712Mhz *\n2: 2400Mhz\n")
    assert bench._read_sclk_mhz(str(f)) == 1712
    f.write_text("S: 96Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench._read_sclk_mhz(str(f)) == 96
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench._read_sclk_mhz(str(f)) is None
    assert bench._read_sclk_mhz(str(tmp_path / "missing")) is None


@pytest.mark.parametrize("m, n, k", [(2048, 4096, 4096),   # 128 tiles of 256 x 256: the chip is not filled
                                     (16, 4096, 11008),    # few tokens: the weight-streaming product
                                     (4096, 4000, 4096),   # n not a multiple of 256
                                     (4096, 4096, 11000)]) # k not a multiple of 64
def test_mfma_ceiling_only_where_the_probe_is_the_products_ceiling(m, n, k):
    """The bench line's MFMA ceiling is measured only where the probe's
    256 x 256 tiles fill the chip; elsewhere the figure is absent, decided
    before anything touches a GPU."""
    assert bench.mfma_ceiling(None, None, None, None, None, m, n, k) is None
