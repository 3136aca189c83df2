"""Build libsq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m w8a8_quantized_linear_sq_amd.build

Each .hip source compiles to an object in ``_build/`` (in parallel), then
one shared library is linked next to this file. The measurement probe
(sq_probe.hip: the int8 matrix units' rate with no memory work, read by the
benchmark's reference mode only) links into a library of its own,
libsq_probe.so. hipcc cross-compiles, so no GPU is needed to build.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsq.so")
PROBE_LIB = os.path.join(PKG, "libsq_probe.so")
SOURCES = ["sq_api.hip", "sq_quant.hip", "sq_gemm.hip", "sq_wo.hip", "sq_error.hip", "sq_ste.hip"]
PROBE_SOURCE = "sq_probe.hip"
ARCH = os.environ.get("SQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # the quantisation steps must round every fp32 operation on its own
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
