"""Host proof of the activation kernel's division scheme for bf16 inputs:
y = RN(1/s), q0 = RN(x y), q1 = fma(fma(-q0, s, x), y, q0) equals the IEEE
quotient RN(x/s) for every binary32 significand of s and every bf16
significand of x (2^30 cases), plus random exponents inside the kernel's
guard 2^-50 <= |q0| <= 2^120. See tests/fastdiv_check.c. (The GPU
test suite extends this to every binary32 numerator significand on the
device itself: test_division_scheme_is_correctly_rounded.)"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fast_division_is_exact_for_bf16(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run(["gcc", "-O2", "-mfma", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "fastdiv_check.c"), "-o", exe, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "exhaustive: 0 mismatches, 0 outside the guard" in r.stdout, r.stdout
    assert "random exponents: 0 mismatches" in r.stdout, r.stdout
