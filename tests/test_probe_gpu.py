"""The measurement probes of libsq_probe.so (the benchmark's MFMA ceiling and
operand-stream reference) on the GPU: each launch succeeds, and the clocks
its workgroups report show the work the figures rest on was done (a loop of
2048 matrix instructions per SIMD at 32 cycles each cannot take fewer than
65536 shader cycles)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV, require_gpu
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import build as hip_build


def _probe():
    P = ctypes.CDLL(hip_build.PROBE_LIB)
    P.sqp_mfma_ceiling.restype = ctypes.c_int
    P.sqp_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.sqp_stream_probe.restype = ctypes.c_int
    P.sqp_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return P


def _codes(rows, k, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-127, 128, (rows, k), dtype=torch.int8, generator=g).to(DEV)


def _check_clocks(clocks, tiles, min_cycles):
    c = clocks.view(tiles, 5).cpu().numpy()
    cycles, ticks = c[:, 0].astype(np.float64), c[:, 1].astype(np.float64)
    assert np.all(ticks > 0), "loop took no 100 MHz ticks"
    assert np.all(cycles >= min_cycles), f"loop shorter than its instructions allow: {cycles.min()} cycles"
    mhz = cycles / (ticks / 100.0)
    assert np.all((mhz > 300) & (mhz < 3000)), f"implausible shader clock {mhz.min()}-{mhz.max()} MHz"
    # entry <= loop start <= loop end on the 100 MHz counter
    assert np.all(c[:, 2] <= c[:, 3]) and np.all(c[:, 3] <= c[:, 4])


@pytest.mark.gpu
@pytest.mark.parametrize("k", [64, 1024])
def test_mfma_ceiling_probe_runs_its_instructions(k):
    require_gpu()
    P = _probe()
    m = n = 512
    tiles = (m // 256) * (n // 256)
    xq, wq = _codes(m, k, 1), _codes(n, k, 2)
    sink = torch.zeros(tiles * 512, dtype=torch.int32, device=DEV)
    clocks = torch.zeros(5 * tiles, dtype=torch.int64, device=DEV)
    print(f"mfma ceiling probe m=n={m} k={k}", flush=True)
    assert P.sqp_mfma_ceiling(xq.data_ptr(), wq.data_ptr(), m, n, k, sink.data_ptr(), clocks.data_ptr(), None) == 0
    torch.cuda.synchronize()
    # per SIMD: 2 wavefronts x 16 instructions per step, 32 cycles each
    _check_clocks(clocks, tiles, 0.95 * 2 * 16 * (k // 64) * 32)
    assert sink.abs().sum().item() > 0, "accumulators all zero on random codes"


@pytest.mark.gpu
@pytest.mark.parametrize("mfma", [0, 1])
def test_operand_stream_probe_runs(mfma):
    require_gpu()
    P = _probe()
    m = n = 512
    k = 1024
    tiles = (m // 256) * (n // 256)
    a, b = B.tiled_empty(m, k, DEV), B.tiled_empty(n, k, DEV)
    a.copy_(_codes(1, a.numel(), 3).view(-1))
    b.copy_(_codes(1, b.numel(), 4).view(-1))
    sink = torch.zeros(tiles * 512, dtype=torch.int32, device=DEV)
    clocks = torch.zeros(5 * tiles, dtype=torch.int64, device=DEV)
    print(f"operand stream probe mfma={mfma} m=n={m} k={k}", flush=True)
    assert P.sqp_stream_probe(a.data_ptr(), b.data_ptr(), m, n, k, mfma, sink.data_ptr(), clocks.data_ptr(),
                              None) == 0
    torch.cuda.synchronize()
    _check_clocks(clocks, tiles, 0.95 * 2 * 16 * (k // 64) * 32 if mfma else 1)
    # each thread folds in a byte its own wavefront loaded into LDS (and,
    # with the matrix instructions, its accumulators): random codes are not
    # all zero
    assert np.any(sink.cpu().numpy() != 0)
