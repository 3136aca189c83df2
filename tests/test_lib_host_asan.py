"""The library's host code (argument checks, launch planning) built with
AddressSanitizer for the host compilation only (the device code is built
as usual and never launched: none of these checks launches a kernel).
Every host ABI check runs against that build without a report (CPU only).
A child Python process preloads clang's AddressSanitizer runtime and points
the binding at the checked build."""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

from w8a8_quantized_linear_sq_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# the sanitizer applies to the host compilation only
FLAGS = (f"--offload-arch={libbuild.ARCH} -O1 -g -std=c++17 -fPIC -ffp-contract=off "
         "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer").split()
LINK = f"--offload-arch={libbuild.ARCH} -shared -fPIC -Xarch_host -fsanitize=address".split()

PLUGIN = """from w8a8_quantized_linear_sq_amd import binding as B

B.LIB_PATH = {lib!r}
"""


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _compile(args):
    src, obj = args
    r = subprocess.run([libbuild.HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-2000:]}")
    return obj


def test_host_abi_checks_under_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(libbuild.HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set in this environment")
    jobs = [(os.path.join(libbuild.CSRC, s), str(tmp_path / (os.path.splitext(s)[0] + ".o"))) for s in libbuild.SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    lib = str(tmp_path / "libsq_host_asan.so")
    r = subprocess.run([libbuild.HIPCC, *LINK, *objs, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms, "the build is not instrumented"
    (tmp_path / "host_asan_lib.py").write_text(PLUGIN.format(lib=lib))
    env = dict(os.environ, PYTHONPATH=f"{tmp_path}{os.pathsep}{ROOT}", LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:exitcode=66")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_host.py"), "-q",
                        "-p", "host_asan_lib", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"exit {r.returncode}\n{out[-4000:]}"
    assert " passed" in r.stdout and "AddressSanitizer" not in out, out[-4000:]
