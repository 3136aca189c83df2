"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
runs every pin once without a report (CPU only): no out-of-bounds access,
use after free, signed overflow, invalid shift or other undefined behaviour
on any pinned input. The sanitizer runtimes are preloaded into a child
Python process that loads the checked build."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import sys
sys.path[:0] = [{here!r}, {root!r}]
import oracle, pins
o = oracle.Oracle({lib!r})
for pin in pins.ALL_PINS:
    pin(o)
print("pins:", len(pins.ALL_PINS))
"""


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = str(tmp_path / "libsq_oracle_sanitized.so")
    oracle.build(lib, sanitize=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=66",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=67",
               OMP_NUM_THREADS="1")
    code = CHILD.format(here=HERE, root=ROOT, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "pins:" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
