"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/sq.h declares, and every argument error returns its status
before anything is launched."""
import ctypes
import subprocess

import pytest

from w8a8_quantized_linear_sq_amd import binding as B

BAD = 0x1001          # a misaligned fake address (never dereferenced)
OK_PTR = 0x10000      # an aligned fake address (never dereferenced)


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_function(L):
    declared = B.header_functions()
    assert set(declared) >= {"sq_calibrate", "sq_prepare_weight", "sq_quantize_act", "sq_w8a8_gemm",
                             "sq_w8a8_linear", "sq_w8a8_linear_workspace_bytes", "sq_status_string",
                             "sq_abi_version", "sq_selfcheck_reciprocal", "sq_selfcheck_division"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        getattr(L, f)


def test_abi_version_and_status_strings(L):
    assert L.sq_abi_version() == 1
    for code in (0, 1, -1, -2, -3, -4, -5, -6):
        s = B.status_string(code)
        assert s.startswith("SQ_"), s
    assert "unknown" in B.status_string(42)


def test_workspace_bytes(L):
    assert L.sq_w8a8_linear_workspace_bytes(0, 64) == 0
    assert L.sq_w8a8_linear_workspace_bytes(3, 16) == 256 + 12
    assert L.sq_w8a8_linear_workspace_bytes(4096, 4096) == 4096 * 4096 + 4 * 4096


def test_calibrate_errors(L):
    f = L.sq_calibrate
    assert f(OK_PTR, 7, 4, 64, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_I32, 4, 64, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_BF16, -1, 64, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, 0, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, B.SQ_MAX_K + 16, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, 24, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(None, B.SQ_BF16, 4, 64, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 4, 64, None, None) == B.SQ_ERR_ARG
    assert f(BAD, B.SQ_BF16, 4, 64, OK_PTR, None) == B.SQ_ERR_ALIGN
    # empty batch: a no-op that needs no pointer at all
    assert f(None, B.SQ_BF16, 0, 64, None, None) == B.SQ_OK


def test_calibrate_batches_errors(L):
    f = L.sq_calibrate_batches

    def call(ptrs, rows, nbatch=None, xt=B.SQ_BF16, k=64, run=OK_PTR, first=0):
        n = len(rows) if nbatch is None else nbatch
        pa = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
        ra = (ctypes.c_int64 * max(len(rows), 1))(*rows)
        return f(pa, ra, n, xt, k, run, first, None)

    two = [OK_PTR, OK_PTR + 4096]
    assert call(two, [4, 4], xt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(two, [4, 4], nbatch=0) == B.SQ_ERR_SHAPE
    assert call(two, [4, 4], nbatch=B.SQ_MAX_CALIB_BATCHES + 1) == B.SQ_ERR_SHAPE
    assert call(two, [4, -1]) == B.SQ_ERR_SHAPE
    assert call(two, [4, 4], k=0) == B.SQ_ERR_SHAPE
    assert call(two, [4, 4], k=B.SQ_MAX_K + 16) == B.SQ_ERR_SHAPE
    assert call(two, [4, 4], k=24) == B.SQ_ERR_ALIGN
    assert call([OK_PTR, 0], [4, 4]) == B.SQ_ERR_ARG
    assert call([OK_PTR, BAD], [4, 4]) == B.SQ_ERR_ALIGN
    assert call(two, [4, 4], run=None) == B.SQ_ERR_ARG
    assert call(two, [4, 4], run=BAD) == B.SQ_ERR_ALIGN
    # rows past the limit, alone or only in sum
    assert call(two, [B.SQ_MAX_ROWS + 1, 0]) == B.SQ_ERR_SHAPE
    assert call(two, [B.SQ_MAX_ROWS, 1]) == B.SQ_ERR_SHAPE
    assert call(two, [1 << 62, 1 << 62]) == B.SQ_ERR_SHAPE
    # null host arrays
    assert f(None, (ctypes.c_int64 * 1)(4), 1, B.SQ_BF16, 64, OK_PTR, 0, None) == B.SQ_ERR_ARG
    assert f((ctypes.c_void_p * 1)(OK_PTR), None, 1, B.SQ_BF16, 64, OK_PTR, 0, None) == B.SQ_ERR_ARG
    # empty batches need no pointer; with no rows at all and first == 0 the
    # call is a no-op
    assert call([0, 0, 0], [0, 0, 0]) == B.SQ_OK


def test_calibrate_batches_binding_checks():
    import torch
    run = torch.zeros(64)
    with pytest.raises(ValueError):
        B.sq_calibrate_batches([], run)
    with pytest.raises(ValueError):
        B.sq_calibrate_batches([torch.zeros(2, 64), torch.zeros(2, 32)], run)
    with pytest.raises(ValueError):
        B.sq_calibrate_batches([torch.zeros(2, 64), torch.zeros(2, 64, dtype=torch.bfloat16)], run)
    with pytest.raises(TypeError):
        B.sq_calibrate_batches([torch.zeros(2, 64)], run.double())


def test_prepare_weight_errors(L):
    f = L.sq_prepare_weight
    args = dict(w=OK_PTR, wt=B.SQ_BF16, n=8, k=64, mx=OK_PTR, alpha=0.5, s=OK_PTR, wq=OK_PTR, ws=OK_PTR)

    def call(**kw):
        a = {**args, **kw}
        return f(a["w"], a["wt"], a["n"], a["k"], a["mx"], a["alpha"], a["s"], a["wq"], a["ws"], None)

    assert call(wt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=-16) == B.SQ_ERR_SHAPE
    assert call(k=40) == B.SQ_ERR_ALIGN
    for a in (-0.01, 1.01, float("nan"), float("inf")):
        assert call(alpha=a) == B.SQ_ERR_ARG
    for key in ("w", "s", "wq", "ws"):
        assert call(**{key: None}) == B.SQ_ERR_ARG
    for key in ("w", "s", "wq", "mx"):
        assert call(**{key: BAD}) == B.SQ_ERR_ALIGN


def test_quantize_act_errors(L):
    f = L.sq_quantize_act
    assert f(OK_PTR, 5, 4, 64, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_BF16, -3, 64, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, 48 + 8, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(OK_PTR, B.SQ_BF16, 4, 64, None, OK_PTR, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 4, 64, OK_PTR, BAD, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(None, B.SQ_BF16, 0, 64, None, None, None, None) == B.SQ_OK


def test_gemm_errors(L):
    f = L.sq_w8a8_gemm

    def call(xq=OK_PTR, sx=OK_PTR, m=4, wq=OK_PTR, sw=OK_PTR, n=8, k=64, bias=None, bt=B.SQ_F32, y=OK_PTR,
             yt=B.SQ_BF16):
        return f(xq, sx, m, wq, sw, n, k, bias, bt, y, yt, None)

    assert call(yt=9) == B.SQ_ERR_DTYPE
    assert call(bias=OK_PTR, bt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(m=-1) == B.SQ_ERR_SHAPE
    assert call(k=8) == B.SQ_ERR_ALIGN
    assert call(xq=None) == B.SQ_ERR_ARG
    assert call(sx=None) == B.SQ_ERR_ARG
    assert call(y=BAD) == B.SQ_ERR_ALIGN
    assert call(m=0, xq=None, y=None) == B.SQ_OK


def test_linear_errors(L):
    f = L.sq_w8a8_linear
    need = L.sq_w8a8_linear_workspace_bytes(4, 64)

    def call(x=OK_PTR, xt=B.SQ_BF16, m=4, k=64, s=OK_PTR, wq=OK_PTR, sw=OK_PTR, n=8, bias=None, y=OK_PTR,
             yt=B.SQ_BF16, ws=OK_PTR, wsb=need):
        return f(x, xt, m, k, s, wq, sw, n, bias, y, yt, ws, wsb, None)

    assert call(xt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(n=-2) == B.SQ_ERR_SHAPE
    assert call(k=72) == B.SQ_ERR_ALIGN
    assert call(x=None) == B.SQ_ERR_ARG
    assert call(s=None) == B.SQ_ERR_ARG
    assert call(ws=None) == B.SQ_ERR_WORKSPACE
    assert call(wsb=need - 1) == B.SQ_ERR_WORKSPACE
    assert call(ws=OK_PTR + 16) == B.SQ_ERR_ALIGN
    assert call(x=BAD) == B.SQ_ERR_ALIGN
    assert call(m=0, x=None, y=None, ws=None, wsb=0) == B.SQ_OK


def test_selfcheck_errors(L):
    assert L.sq_selfcheck_reciprocal(None, None) == B.SQ_ERR_ARG
    assert L.sq_selfcheck_reciprocal(OK_PTR + 4, None) == B.SQ_ERR_ALIGN
    assert L.sq_selfcheck_division(0, 16, None, None) == B.SQ_ERR_ARG
    assert L.sq_selfcheck_division(0, 16, OK_PTR + 4, None) == B.SQ_ERR_ALIGN
    assert L.sq_selfcheck_division(8, 4, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert L.sq_selfcheck_division(0, (1 << 23) + 1, OK_PTR, None) == B.SQ_ERR_SHAPE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_prepared_call_keeps_its_buffers_alive(L):
    """A prepared call holds only raw pointers for the C call, so it must keep
    the tensors behind them referenced: freed and returned to the device, they
    would leave a captured launch pointing at unmapped memory. Marshalled
    only, never invoked here."""
    import gc
    import weakref

    import torch

    x = torch.zeros(4, 64)
    run = torch.zeros(64)
    refs = [weakref.ref(x), weakref.ref(run)]
    call = B.prepared(B.sq_calibrate, x, run)
    del x, run
    gc.collect()
    assert all(r() is not None for r in refs)
    del call
    gc.collect()
    assert all(r() is None for r in refs)


def test_quantize_tensor_errors(L):
    f = L.sq_quantize_tensor
    assert f(OK_PTR, B.SQ_I32, 64, OK_PTR, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_BF16, 0, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, -16, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 40, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(None, B.SQ_BF16, 64, OK_PTR, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 64, None, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 64, OK_PTR, None, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 64, BAD, OK_PTR, None) == B.SQ_ERR_ALIGN


def test_gemm_per_tensor_errors(L):
    f = L.sq_w8a8_gemm_per_tensor
    args = dict(xq=OK_PTR, sx=OK_PTR, m=4, wq=OK_PTR, sw=OK_PTR, n=8, k=64, bias=None, bt=B.SQ_F32, y=OK_PTR,
                yt=B.SQ_F32)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["xq"], a["sx"], a["m"], a["wq"], a["sw"], a["n"], a["k"], a["bias"], a["bt"], a["y"], a["yt"], None)

    assert call(yt=9) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=8) == B.SQ_ERR_ALIGN
    assert call(sw=None) == B.SQ_ERR_ARG
    assert call(y=BAD) == B.SQ_ERR_ALIGN
    assert call(m=0) == B.SQ_OK  # nothing to do, nothing launched


def test_wo_linear_errors(L):
    f = L.sq_wo_linear

    def call(x=OK_PTR, xt=B.SQ_BF16, m=4, k=64, wq=OK_PTR, sw=OK_PTR, n=8, bias=None, bt=B.SQ_F32, y=OK_PTR,
             yt=B.SQ_BF16):
        return f(x, xt, m, k, wq, sw, n, bias, bt, y, yt, None)

    assert call(xt=B.SQ_F32) == B.SQ_ERR_DTYPE   # bf16 activations only
    assert call(yt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(bias=OK_PTR, bt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=40) == B.SQ_ERR_ALIGN
    assert call(sw=None) == B.SQ_ERR_ARG
    assert call(x=BAD) == B.SQ_ERR_ALIGN
    assert call(m=0, x=None) == B.SQ_OK


def test_weight_col_max_errors(L):
    f = L.sq_weight_col_max
    assert f(OK_PTR, B.SQ_I32, 4, 64, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_BF16, 0, 64, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, 40, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(None, B.SQ_BF16, 4, 64, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 4, 64, None, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 4, 64, BAD, None) == B.SQ_ERR_ALIGN


def test_recompute_smooth_scale_errors(L):
    f = L.sq_recompute_smooth_scale

    def call(w=OK_PTR, wt=B.SQ_BF16, n=4, k=64, mx=OK_PTR, mw=OK_PTR, alpha=0.5, s=OK_PTR, wq=OK_PTR, sw=OK_PTR):
        return f(w, wt, n, k, mx, mw, alpha, s, wq, sw, None)

    assert call(wt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=8) == B.SQ_ERR_ALIGN
    assert call(alpha=1.5) == B.SQ_ERR_ARG
    assert call(alpha=float("nan")) == B.SQ_ERR_ARG
    assert call(mw=None) == B.SQ_ERR_ARG          # calibrated needs the stored weight max
    assert call(s=None) == B.SQ_ERR_ARG
    assert call(mw=BAD) == B.SQ_ERR_ALIGN
    assert call(wq=BAD) == B.SQ_ERR_ALIGN


def test_reference_linear_errors(L):
    f = L.sq_reference_linear

    def call(x=OK_PTR, xt=B.SQ_BF16, m=4, k=64, w=OK_PTR, n=8, bias=None, bt=B.SQ_F32, y=OK_PTR, yt=B.SQ_F32):
        return f(x, xt, m, k, w, n, bias, bt, y, yt, None)

    assert call(xt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(yt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(bias=OK_PTR, bt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=B.SQ_MAX_K + 16) == B.SQ_ERR_SHAPE
    assert call(k=20) == B.SQ_ERR_ALIGN
    assert call(w=None) == B.SQ_ERR_ARG
    assert call(y=BAD) == B.SQ_ERR_ALIGN
    assert call(m=0, x=None, w=None, y=None) == B.SQ_OK


def test_relative_error_errors(L):
    f = L.sq_relative_error
    need = L.sq_relative_error_workspace_bytes(1000)
    assert need >= 16 and need % 16 == 0
    assert L.sq_relative_error_workspace_bytes(0) == 0
    # more elements never need fewer partial sums, and the block count is capped
    assert L.sq_relative_error_workspace_bytes(10 ** 9) >= need
    assert L.sq_relative_error_workspace_bytes(10 ** 12) == L.sq_relative_error_workspace_bytes(10 ** 11)
    assert f(OK_PTR, OK_PTR, 0, OK_PTR, need, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(None, OK_PTR, 1000, OK_PTR, need, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, OK_PTR, 1000, OK_PTR, need, None, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, OK_PTR, 1000, None, need, OK_PTR, None) == B.SQ_ERR_WORKSPACE
    assert f(OK_PTR, OK_PTR, 1000, OK_PTR, need - 1, OK_PTR, None) == B.SQ_ERR_WORKSPACE
    assert f(BAD, OK_PTR, 1000, OK_PTR, need, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(OK_PTR, OK_PTR, 1000, OK_PTR, need, OK_PTR + 4, None) == B.SQ_ERR_ALIGN


def test_smoothing_factor_errors(L):
    f = L.sq_smoothing_factor
    assert f(OK_PTR, OK_PTR, 0.5, 0, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, OK_PTR, 0.5, 40, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(OK_PTR, OK_PTR, -0.1, 64, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, None, 0.5, 64, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, OK_PTR, 0.5, 64, None, None) == B.SQ_ERR_ARG
    assert f(BAD, OK_PTR, 0.5, 64, OK_PTR, None) == B.SQ_ERR_ALIGN


def test_quantize_weight_errors(L):
    f = L.sq_quantize_weight
    assert f(OK_PTR, B.SQ_I32, 4, 64, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_BF16, 0, 64, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, 72, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(OK_PTR, B.SQ_BF16, 4, 64, None, OK_PTR, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 4, 64, OK_PTR, BAD, OK_PTR, None) == B.SQ_ERR_ALIGN


def test_tiled_bytes(L):
    # rows padded to 16, k to a multiple of 64
    assert L.sq_tiled_bytes(0, 64) == 0
    assert L.sq_tiled_bytes(4, 0) == 0
    assert L.sq_tiled_bytes(1, 16) == 16 * 64
    assert L.sq_tiled_bytes(17, 80) == 32 * 128
    assert L.sq_tiled_bytes(4096, 4096) == 4096 * 4096
    assert L.sq_tiled_bytes(4096, 11008) == 4096 * 11008  # 11008 = 172 * 64
    assert L.sq_tiled_bytes(333, 4000) == 336 * 4032


def test_untile_matches_the_layout_formula():
    import torch
    rows, k = 19, 80
    r16, k64 = 32, 128
    flat = torch.arange(r16 * k64, dtype=torch.int64)
    a = B.untile(flat, rows, k)
    for i in (0, 1, 15, 16, 18):
        for j in (0, 5, 63, 64, 79):
            assert a[i, j] == ((i // 16) * (k64 // 64) + j // 64) * 1024 + (i % 16) * 64 + j % 64


def test_tiled_entry_errors(L):
    f = L.sq_quantize_act_tiled
    assert f(OK_PTR, 5, 4, 64, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert f(OK_PTR, B.SQ_BF16, -3, 64, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert f(OK_PTR, B.SQ_BF16, 4, 56, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(OK_PTR, B.SQ_BF16, 4, 64, None, OK_PTR, OK_PTR, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, B.SQ_BF16, 4, 64, OK_PTR, BAD, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert f(None, B.SQ_BF16, 0, 64, None, None, None, None) == B.SQ_OK

    g = L.sq_prepare_weight_tiled
    assert g(OK_PTR, B.SQ_I32, 8, 64, OK_PTR, 0.5, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert g(OK_PTR, B.SQ_BF16, 0, 64, OK_PTR, 0.5, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert g(OK_PTR, B.SQ_BF16, 8, 40, OK_PTR, 0.5, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert g(OK_PTR, B.SQ_BF16, 8, 64, OK_PTR, 1.5, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_ARG
    assert g(OK_PTR, B.SQ_BF16, 8, 64, OK_PTR, 0.5, OK_PTR, None, OK_PTR, None) == B.SQ_ERR_ARG
    assert g(OK_PTR, B.SQ_BF16, 8, 64, BAD, 0.5, OK_PTR, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN

    h = L.sq_w8a8_gemm_tiled

    def call(xq=OK_PTR, sx=OK_PTR, m=4, wq=OK_PTR, sw=OK_PTR, n=8, k=64, bias=None, bt=B.SQ_F32, y=OK_PTR,
             yt=B.SQ_BF16):
        return h(xq, sx, m, wq, sw, n, k, bias, bt, y, yt, None)

    assert call(yt=9) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=8) == B.SQ_ERR_ALIGN
    assert call(wq=None) == B.SQ_ERR_ARG
    assert call(y=BAD) == B.SQ_ERR_ALIGN
    assert call(m=0, xq=None, y=None) == B.SQ_OK

    w = L.sq_wo_linear_tiled
    assert w(OK_PTR, B.SQ_F32, 4, 64, OK_PTR, OK_PTR, 8, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_DTYPE
    assert w(OK_PTR, B.SQ_BF16, 4, 64, OK_PTR, OK_PTR, 8, None, B.SQ_F32, OK_PTR, B.SQ_I32, None) == B.SQ_ERR_DTYPE
    assert w(OK_PTR, B.SQ_BF16, 4, 64, OK_PTR, OK_PTR, 0, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
    assert w(OK_PTR, B.SQ_BF16, 4, 40, OK_PTR, OK_PTR, 8, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_ALIGN
    assert w(OK_PTR, B.SQ_BF16, 4, 64, None, OK_PTR, 8, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_ARG
    assert w(OK_PTR, B.SQ_BF16, 4, 64, BAD, OK_PTR, 8, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_ALIGN
    assert w(None, B.SQ_BF16, 0, 64, None, None, 8, None, B.SQ_F32, None, B.SQ_BF16, None) == B.SQ_OK

    t = L.sq_quantize_tensor_tiled
    assert t(OK_PTR, B.SQ_I32, 4, 64, OK_PTR, OK_PTR, None) == B.SQ_ERR_DTYPE
    assert t(OK_PTR, B.SQ_BF16, 0, 64, OK_PTR, OK_PTR, None) == B.SQ_ERR_SHAPE
    assert t(OK_PTR, B.SQ_BF16, 4, 40, OK_PTR, OK_PTR, None) == B.SQ_ERR_ALIGN
    assert t(OK_PTR, B.SQ_BF16, 4, 64, None, OK_PTR, None) == B.SQ_ERR_ARG
    assert t(OK_PTR, B.SQ_BF16, 4, 64, BAD, OK_PTR, None) == B.SQ_ERR_ALIGN
    p = L.sq_w8a8_gemm_per_tensor_tiled
    assert p(OK_PTR, OK_PTR, 4, OK_PTR, OK_PTR, 8, 64, None, B.SQ_F32, OK_PTR, 9, None) == B.SQ_ERR_DTYPE
    assert p(OK_PTR, OK_PTR, 4, OK_PTR, OK_PTR, 0, 64, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
    assert p(None, OK_PTR, 4, OK_PTR, OK_PTR, 8, 64, None, B.SQ_F32, OK_PTR, B.SQ_BF16, None) == B.SQ_ERR_ARG


def test_tiled_layout_roundtrip_random_shapes(L):
    """For random shapes: placing every element at the layout formula's
    address and reading it back with binding.untile is the identity, the
    placements never collide, and they fill exactly sq_tiled_bytes minus the
    padding (host only)."""
    import numpy as np
    import torch
    rng = np.random.default_rng(5)
    for _ in range(40):
        rows = int(rng.integers(1, 70))
        k = int(rng.integers(1, 40)) * 16
        size = L.sq_tiled_bytes(rows, k)
        r16, k64 = (rows + 15) // 16 * 16, (k + 63) // 64 * 64
        assert size == r16 * k64
        a = rng.integers(-128, 128, size=(rows, k)).astype(np.int8)
        i, j = np.meshgrid(np.arange(rows), np.arange(k), indexing="ij")
        addr = ((i // 16) * (k64 // 64) + j // 64) * 1024 + (i % 16) * 64 + j % 64
        assert len(np.unique(addr)) == rows * k and addr.max() < size
        flat = np.zeros(size, np.int8)
        flat[addr] = a
        back = B.untile(torch.from_numpy(flat), rows, k).numpy()
        assert np.array_equal(back, a)


def test_size_limits(L):
    """Row counts above SQ_MAX_ROWS, and products with more than
    SQ_MAX_TILES output tiles of 128 x 128, return SQ_ERR_SHAPE before
    anything is launched (the kernels count rows and tiles in int32)."""
    big, over = B.SQ_MAX_ROWS, B.SQ_MAX_ROWS + 1
    P = OK_PTR
    assert L.sq_calibrate(P, B.SQ_BF16, over, 64, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_calibrate(P, B.SQ_BF16, 1 << 31, 64, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_prepare_weight(P, B.SQ_BF16, over, 64, P, 0.5, P, P, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_prepare_weight_tiled(P, B.SQ_BF16, 1 << 31, 64, P, 0.5, P, P, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_quantize_act(P, B.SQ_BF16, over, 64, P, P, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_quantize_act_tiled(P, B.SQ_BF16, 1 << 31, 64, P, P, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_weight_col_max(P, B.SQ_BF16, over, 64, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_quantize_weight(P, B.SQ_BF16, over, 64, P, P, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_recompute_smooth_scale(P, B.SQ_BF16, over, 64, P, P, 0.5, P, P, P, None) == B.SQ_ERR_SHAPE
    assert L.sq_quantize_tensor_tiled(P, B.SQ_BF16, over, 64, P, P, None) == B.SQ_ERR_SHAPE
    for fn in (L.sq_w8a8_gemm, L.sq_w8a8_gemm_tiled, L.sq_w8a8_gemm_per_tensor, L.sq_w8a8_gemm_per_tensor_tiled):
        # 2^31 tokens or channels (the value that wrapped negative in int32)
        assert fn(P, P, 1 << 31, P, P, 8, 64, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
        assert fn(P, P, 8, P, P, 1 << 31, 64, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
        assert fn(P, P, 4, P, P, over, 64, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
        # each size allowed, the output too large for the tile grid
        assert fn(P, P, big, P, P, big, 64, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
        side = 128 * 2897                     # 2897^2 = 8392609 > 2^23 - 1 tiles
        assert fn(P, P, side, P, P, side, 64, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
    for fn in (L.sq_wo_linear, L.sq_wo_linear_tiled):
        assert fn(P, B.SQ_BF16, 4, 64, P, P, 1 << 31, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
        assert fn(P, B.SQ_BF16, over, 64, P, P, 8, None, B.SQ_F32, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
    assert L.sq_reference_linear(P, B.SQ_BF16, big, 64, P, big, None, B.SQ_F32, P, B.SQ_F32,
                                 None) == B.SQ_ERR_SHAPE
    ws = L.sq_w8a8_linear_workspace_bytes(4, 64)
    assert L.sq_w8a8_linear(P, B.SQ_BF16, 4, 64, P, P, P, 1 << 31, None, P, B.SQ_BF16, P, ws,
                            None) == B.SQ_ERR_SHAPE


def test_alpha_from_eta_matches_oracle(L, orc):
    """The library's host sigmoid and initial eta equal the oracle's bit for
    bit (both binary64 rounded once to binary32)."""
    import numpy as np
    for eta in np.linspace(-12.0, 12.0, 241, dtype=np.float32):
        assert np.float32(L.sq_alpha_from_eta(float(eta))) == orc.alpha_from_eta(float(eta)), eta
    for a in (1e-7, 0.05, 0.25, 0.5, 0.75, 0.9, 1.0):
        assert np.float32(L.sq_eta_from_alpha(a)) == orc.eta_from_alpha(a), a
    assert L.sq_alpha_from_eta(0.0) == 0.5


def test_ste_backward_errors(L):
    f = L.sq_ste_backward
    need = L.sq_ste_backward_workspace_bytes(8, 6, 64)
    assert need > 0 and L.sq_ste_backward_workspace_bytes(0, 6, 64) == 0

    def call(dy=OK_PTR, dyt=B.SQ_F32, m=8, n=6, k=64, x=OK_PTR, xt=B.SQ_BF16, w=OK_PTR, wt=B.SQ_BF16, s=OK_PTR,
             xq=OK_PTR, sx=OK_PTR, wq=OK_PTR, sw=OK_PTR, mx=OK_PTR, mw=OK_PTR, alpha=0.5, dx=OK_PTR, dw=OK_PTR,
             db=None, ds=None, da=OK_PTR, ws=OK_PTR, wsb=need):
        return f(dy, dyt, m, n, k, x, xt, w, wt, s, xq, sx, wq, sw, mx, mw, alpha, dx, dw, db, ds, da, ws, wsb, None)

    assert call(dyt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(xt=7) == B.SQ_ERR_DTYPE
    assert call(m=0) == B.SQ_ERR_SHAPE
    assert call(n=B.SQ_STE_MAX_ROWS + 1) == B.SQ_ERR_SHAPE
    assert call(k=40) == B.SQ_ERR_ALIGN
    assert call(alpha=1.5) == B.SQ_ERR_ARG
    for key in ("dy", "x", "w", "s", "xq", "sx", "wq", "sw", "dx", "dw", "da"):
        assert call(**{key: None}) == B.SQ_ERR_ARG, key
    assert call(mw=None) == B.SQ_ERR_ARG
    assert call(ws=None) == B.SQ_ERR_WORKSPACE
    assert call(wsb=need - 1) == B.SQ_ERR_WORKSPACE
    for key in ("x", "w", "xq", "wq", "dx", "dw"):
        assert call(**{key: BAD}) == B.SQ_ERR_ALIGN, key
    assert call(ws=OK_PTR + 16) == B.SQ_ERR_ALIGN


def test_aux_loss_grad_errors(L):
    f = L.sq_aux_loss_grad
    need = L.sq_aux_loss_grad_workspace_bytes(100)
    assert f(OK_PTR, OK_PTR, 0, OK_PTR, OK_PTR, OK_PTR, need, None) == B.SQ_ERR_SHAPE
    assert f(None, OK_PTR, 100, OK_PTR, OK_PTR, OK_PTR, need, None) == B.SQ_ERR_ARG
    assert f(OK_PTR, OK_PTR, 100, OK_PTR, OK_PTR, OK_PTR, need - 1, None) == B.SQ_ERR_WORKSPACE
    assert f(BAD, OK_PTR, 100, OK_PTR, OK_PTR, OK_PTR, need, None) == B.SQ_ERR_ALIGN


@pytest.mark.parametrize("fused", [False, True])
def test_linear_tiled_errors(L, fused):
    f = L.sq_w8a8_linear_tiled_fused if fused else L.sq_w8a8_linear_tiled
    need = (L.sq_w8a8_linear_tiled_fused_workspace_bytes if fused else L.sq_w8a8_linear_tiled_workspace_bytes)(4, 64)
    assert need >= (1024 if fused else 0) + 16 * 64 + 16
    assert L.sq_w8a8_linear_tiled_workspace_bytes(0, 64) == 0
    if fused:
        big = L.sq_w8a8_linear_tiled_fused_workspace_bytes(65, 64)
        assert f(OK_PTR, B.SQ_BF16, 65, 64, OK_PTR, OK_PTR, OK_PTR, 8, None, B.SQ_F32, OK_PTR, B.SQ_BF16, OK_PTR,
                 big, None) == B.SQ_ERR_SHAPE

    def call(x=OK_PTR, xt=B.SQ_BF16, m=4, k=64, s=OK_PTR, wq=OK_PTR, sw=OK_PTR, n=8, bias=None, bt=B.SQ_F32,
             y=OK_PTR, yt=B.SQ_BF16, ws=OK_PTR, wsb=need):
        return f(x, xt, m, k, s, wq, sw, n, bias, bt, y, yt, ws, wsb, None)

    assert call(xt=B.SQ_I32) == B.SQ_ERR_DTYPE
    assert call(bias=OK_PTR, bt=9) == B.SQ_ERR_DTYPE
    assert call(n=0) == B.SQ_ERR_SHAPE
    assert call(k=40) == B.SQ_ERR_ALIGN
    assert call(x=None) == B.SQ_ERR_ARG
    assert call(s=None) == B.SQ_ERR_ARG
    assert call(ws=None) == B.SQ_ERR_WORKSPACE
    assert call(wsb=need - 1) == B.SQ_ERR_WORKSPACE
    assert call(ws=OK_PTR + 16) == B.SQ_ERR_ALIGN
    assert call(m=0, x=None, y=None) == B.SQ_OK


def test_mfma_probe_rejects_shapes_before_launch():
    """The measurement probe (libsq_probe.so, the benchmark's MFMA-ceiling
    reference) refuses shapes its grid does not cover, with no launch."""
    from w8a8_quantized_linear_sq_amd import build as hip_build
    P = ctypes.CDLL(hip_build.PROBE_LIB)
    P.sqp_mfma_ceiling.restype = ctypes.c_int
    P.sqp_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for m, n, k in ((255, 256, 64), (256, 300, 64), (256, 256, 32), (256, 256, 96), (0, 256, 64),
                    (1 << 40, 256, 64), (256, 256, 1 << 31)):
        assert P.sqp_mfma_ceiling(OK_PTR, OK_PTR, m, n, k, OK_PTR, OK_PTR, None) == -1, (m, n, k)
    P.sqp_stream_probe.restype = ctypes.c_int
    P.sqp_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for m, n, k in ((255, 256, 64), (256, 300, 64), (256, 256, 32), (256, 256, 96), (0, 256, 64),
                    (1 << 40, 256, 64), (256, 256, 1 << 28)):
        for mfma in (0, 1):
            assert P.sqp_stream_probe(OK_PTR, OK_PTR, m, n, k, mfma, OK_PTR, OK_PTR, None) == -1, (m, n, k)
