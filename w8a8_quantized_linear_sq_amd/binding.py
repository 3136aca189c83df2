"""ctypes binding of libsq.so (the C ABI in include/sq.h).

Argument marshalling only: every step of the SmoothQuant W8A8 path runs in
the HIP kernels behind the ABI. torch supplies device memory (``data_ptr``)
and the stream (``torch.cuda.current_stream().cuda_stream``). The functions
keep the ABI's names; sizes are read from the tensors' shapes.

If libsq.so is missing this module raises at first use: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsq.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "sq.h")

SQ_OK, SQ_WARN_UNCALIBRATED = 0, 1
SQ_ERR_ARG, SQ_ERR_SHAPE, SQ_ERR_DTYPE, SQ_ERR_ALIGN, SQ_ERR_WORKSPACE, SQ_ERR_HIP = -1, -2, -3, -4, -5, -6
SQ_F32, SQ_BF16, SQ_I32 = 0, 1, 2
SQ_MAX_K = 16384
SQ_MAX_ROWS = 1 << 30
SQ_MAX_TILES = (1 << 23) - 1
SQ_MAX_CALIB_BATCHES = 8
SQ_NOALLOC_MAX_CODES = 1 << 24
SQ_NOALLOC_MAX_TOKENS = 1 << 14
SQ_STE_MAX_ROWS = 1 << 24


class SQError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


_P, _I64, _SZ, _F, _E = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_int

_SIGNATURES = {
    "sq_calibrate": ([_P, _E, _I64, _I64, _P, _P], _E),
    "sq_calibrate_first": ([_P, _E, _I64, _I64, _P, _P], _E),
    "sq_calibrate_batches": ([_P, _P, _E, _E, _I64, _P, _E, _P], _E),
    "sq_prepare_weight": ([_P, _E, _I64, _I64, _P, _F, _P, _P, _P, _P], _E),
    "sq_quantize_act": ([_P, _E, _I64, _I64, _P, _P, _P, _P], _E),
    "sq_w8a8_gemm": ([_P, _P, _I64, _P, _P, _I64, _I64, _P, _E, _P, _E, _P], _E),
    "sq_w8a8_linear": ([_P, _E, _I64, _I64, _P, _P, _P, _I64, _P, _P, _E, _P, _SZ, _P], _E),
    "sq_w8a8_linear_workspace_bytes": ([_I64, _I64], _SZ),
    "sq_w8a8_linear_noalloc": ([_P, _E, _I64, _I64, _P, _P, _P, _I64, _P, _P, _E, _P], _E),
    "sq_w8a8_linear_tiled_workspace_bytes": ([_I64, _I64], _SZ),
    "sq_w8a8_linear_tiled": ([_P, _E, _I64, _I64, _P, _P, _P, _I64, _P, _E, _P, _E, _P, _SZ, _P], _E),
    "sq_w8a8_linear_tiled_fused_workspace_bytes": ([_I64, _I64], _SZ),
    "sq_w8a8_linear_tiled_fused": ([_P, _E, _I64, _I64, _P, _P, _P, _I64, _P, _E, _P, _E, _P, _SZ, _P], _E),
    "sq_set_fused_wait_polls": ([ctypes.c_int], None),
    "sq_alpha_from_eta": ([_F], _F),
    "sq_eta_from_alpha": ([ctypes.c_double], _F),
    "sq_ste_backward_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "sq_ste_backward": ([_P, _E, _I64, _I64, _I64, _P, _E, _P, _E, _P, _P, _P, _P, _P, _P, _P, _F, _P, _P, _P,
                         _P, _P, _P, _SZ, _P], _E),
    "sq_aux_loss_grad_workspace_bytes": ([_I64], _SZ),
    "sq_aux_loss_grad": ([_P, _P, _I64, _P, _P, _P, _SZ, _P], _E),
    "sq_status_string": ([_E], ctypes.c_char_p),
    "sq_abi_version": ([], _E),
    "sq_quantize_tensor": ([_P, _E, _I64, _P, _P, _P], _E),
    "sq_w8a8_gemm_per_tensor": ([_P, _P, _I64, _P, _P, _I64, _I64, _P, _E, _P, _E, _P], _E),
    "sq_quantize_tensor_tiled": ([_P, _E, _I64, _I64, _P, _P, _P], _E),
    "sq_w8a8_gemm_per_tensor_tiled": ([_P, _P, _I64, _P, _P, _I64, _I64, _P, _E, _P, _E, _P], _E),
    "sq_wo_linear": ([_P, _E, _I64, _I64, _P, _P, _I64, _P, _E, _P, _E, _P], _E),
    "sq_wo_linear_tiled": ([_P, _E, _I64, _I64, _P, _P, _I64, _P, _E, _P, _E, _P], _E),
    "sq_weight_col_max": ([_P, _E, _I64, _I64, _P, _P], _E),
    "sq_recompute_smooth_scale": ([_P, _E, _I64, _I64, _P, _P, _F, _P, _P, _P, _P], _E),
    "sq_smoothing_factor": ([_P, _P, _F, _I64, _P, _P], _E),
    "sq_tiled_bytes": ([_I64, _I64], _SZ),
    "sq_prepare_weight_tiled": ([_P, _E, _I64, _I64, _P, _F, _P, _P, _P, _P], _E),
    "sq_quantize_act_tiled": ([_P, _E, _I64, _I64, _P, _P, _P, _P], _E),
    "sq_w8a8_gemm_tiled": ([_P, _P, _I64, _P, _P, _I64, _I64, _P, _E, _P, _E, _P], _E),
    "sq_quantize_weight": ([_P, _E, _I64, _I64, _P, _P, _P, _P], _E),
    "sq_reference_linear": ([_P, _E, _I64, _I64, _P, _I64, _P, _E, _P, _E, _P], _E),
    "sq_relative_error": ([_P, _P, _I64, _P, _SZ, _P, _P], _E),
    "sq_relative_error_workspace_bytes": ([_I64], _SZ),
    "sq_selfcheck_reciprocal": ([_P, _P], _E),
    "sq_selfcheck_division": ([ctypes.c_uint, ctypes.c_uint, _P, _P], _E),
}

_lib: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """The loaded libsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m w8a8_quantized_linear_sq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/sq.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().sq_status_string(status).decode()


def _check(fn: str, status: int) -> int:
    if status < 0:
        raise SQError(fn, status, status_string(status))
    return status


class _Capture(threading.local):
    on = False
    call = None


_capture = _Capture()


def _invoke(name: str, *args):
    """Calls the C entry point, or records the marshalled call for prepared()."""
    if _capture.on:
        _capture.call = (name, args)
        return SQ_OK
    return _check(name, getattr(lib(), name)(*args))


def prepared(fn, *args, **kwargs):
    """Marshals one call of a wrapper below once and returns a zero-argument
    callable that repeats exactly that C call (same pointers, sizes and
    stream) and checks its status: for launch loops where the per-call
    Python work would otherwise be paced against the GPU. The callable holds
    references to the arguments, so the buffers behind those pointers live as
    long as it does (a graph captured from it needs the callable kept too)."""
    _capture.on = True
    try:
        fn(*args, **kwargs)
        name, cargs = _capture.call
    finally:
        _capture.on = False
        _capture.call = None
    cfn = getattr(lib(), name)

    def call():
        status = cfn(*cargs)
        if status < 0:
            raise SQError(name, status, status_string(status))
        return status

    call.args = (args, kwargs)
    return call


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SQ_F32
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    if t.dtype == torch.int32:
        return SQ_I32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsq must be contiguous")
    return t.data_ptr() or None


def _stream(stream, t: torch.Tensor):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _need_dtype(t: torch.Tensor, dt, what):
    if t.dtype != dt:
        raise TypeError(f"{what} must be {dt}, got {t.dtype}")


# ---------------------------------------------------------------------------
# the ABI, one wrapper per entry point
# ---------------------------------------------------------------------------
def sq_calibrate(x: torch.Tensor, running_max_abs: torch.Tensor, stream=None) -> int:
    """running_max_abs[j] = max(running_max_abs[j], max_r |x[r, j]|)."""
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    _need_dtype(running_max_abs, torch.float32, "running_max_abs")
    return _invoke("sq_calibrate", _ptr(x), _dtype_code(x), rows, k, _ptr(running_max_abs),
                   _stream(stream, x))


def sq_calibrate_first(x: torch.Tensor, running_max_abs: torch.Tensor, stream=None) -> int:
    """running_max_abs[j] = max_r |x[r, j]| (a first batch; no zero fill needed)."""
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    _need_dtype(running_max_abs, torch.float32, "running_max_abs")
    return _invoke("sq_calibrate_first", _ptr(x), _dtype_code(x), rows, k, _ptr(running_max_abs),
                   _stream(stream, running_max_abs))


def sq_calibrate_batches(xs, running_max_abs: torch.Tensor, first: bool = False, stream=None) -> int:
    """Every batch of ``xs`` (a sequence of tensors of one dtype and last
    dimension k) folded into running_max_abs at once; with ``first`` the
    running max starts from these batches alone (no zero fill needed)."""
    xs = list(xs)
    if not xs:
        raise ValueError("sq_calibrate_batches needs at least one batch")
    k = xs[0].shape[-1]
    for x in xs:
        if x.shape[-1] != k or x.dtype != xs[0].dtype:
            raise ValueError("calibration batches must share their dtype and last dimension")
    _need_dtype(running_max_abs, torch.float32, "running_max_abs")
    rows = [x.numel() // k if k else 0 for x in xs]
    ptrs = (ctypes.c_void_p * len(xs))(*[_ptr(x) for x in xs])
    counts = (ctypes.c_int64 * len(xs))(*rows)
    return _invoke("sq_calibrate_batches", ptrs, counts, len(xs), _dtype_code(xs[0]), k, _ptr(running_max_abs),
                   1 if first else 0, _stream(stream, running_max_abs))


def sq_prepare_weight(w: torch.Tensor, x_max_abs: torch.Tensor | None, alpha: float, smooth: torch.Tensor,
                      w_q: torch.Tensor, w_scale: torch.Tensor, stream=None) -> int:
    """s, int8 weights and per-output-channel scales (SQ_WARN_UNCALIBRATED
    when x_max_abs is None)."""
    n, k = w.shape
    _need_dtype(smooth, torch.float32, "smooth")
    _need_dtype(w_q, torch.int8, "w_q")
    _need_dtype(w_scale, torch.float32, "w_scale")
    if x_max_abs is not None:
        _need_dtype(x_max_abs, torch.float32, "x_max_abs")
    return _invoke("sq_prepare_weight", _ptr(w), _dtype_code(w), n, k, _ptr(x_max_abs), float(alpha),
                   _ptr(smooth), _ptr(w_q), _ptr(w_scale), _stream(stream, w))


def sq_quantize_act(x: torch.Tensor, smooth: torch.Tensor, x_q: torch.Tensor, x_scale: torch.Tensor,
                    stream=None) -> int:
    """Per-token int8 codes and scales of x / smooth."""
    m, k = x.shape
    _need_dtype(x_q, torch.int8, "x_q")
    _need_dtype(x_scale, torch.float32, "x_scale")
    return _invoke("sq_quantize_act", _ptr(x), _dtype_code(x), m, k, _ptr(smooth), _ptr(x_q), _ptr(x_scale),
                   _stream(stream, x))


def sq_w8a8_gemm(x_q: torch.Tensor, x_scale: torch.Tensor | None, w_q: torch.Tensor,
                 w_scale: torch.Tensor | None, bias: torch.Tensor | None, y: torch.Tensor, stream=None) -> int:
    """y = x_q w_q^T (int32), dequantised unless y is int32."""
    m, k = x_q.shape
    n = w_q.shape[0]
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_w8a8_gemm", _ptr(x_q), _ptr(x_scale), m, _ptr(w_q), _ptr(w_scale), n, k, _ptr(bias), bt,
                   _ptr(y), _dtype_code(y), _stream(stream, x_q))


def sq_quantize_tensor(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None) -> int:
    """Per-tensor int8 codes of x (any shape, contiguous) and its one scale."""
    _need_dtype(q, torch.int8, "q")
    _need_dtype(scale, torch.float32, "scale")
    if q.numel() != x.numel() or scale.numel() < 1:
        raise ValueError("q must have x's size and scale at least one element")
    return _invoke("sq_quantize_tensor", _ptr(x), _dtype_code(x), x.numel(), _ptr(q), _ptr(scale),
                   _stream(stream, x))


def sq_w8a8_gemm_per_tensor(x_q: torch.Tensor, x_scale: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                            bias: torch.Tensor | None, y: torch.Tensor, stream=None) -> int:
    """y = x_q w_q^T * x_scale[0] * w_scale[0] (+ bias)."""
    m, k = x_q.shape
    n = w_q.shape[0]
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_w8a8_gemm_per_tensor", _ptr(x_q), _ptr(x_scale), m, _ptr(w_q), _ptr(w_scale), n, k,
                   _ptr(bias), bt, _ptr(y), _dtype_code(y), _stream(stream, x_q))


def sq_quantize_tensor_tiled(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None) -> int:
    """Per-tensor int8 codes of a [rows][k] x into 16 x 64 tiles (flat int8 q)
    and its one scale."""
    rows, k = x.shape
    _need_tiled(q, rows, k, "q")
    _need_dtype(scale, torch.float32, "scale")
    return _invoke("sq_quantize_tensor_tiled", _ptr(x), _dtype_code(x), rows, k, _ptr(q), _ptr(scale),
                   _stream(stream, x))


def sq_w8a8_gemm_per_tensor_tiled(x_q: torch.Tensor, x_scale: torch.Tensor, m: int, w_q: torch.Tensor,
                                  w_scale: torch.Tensor, n: int, k: int, bias: torch.Tensor | None, y: torch.Tensor,
                                  stream=None) -> int:
    """sq_w8a8_gemm_per_tensor on operands in 16 x 64 tiles (flat int8)."""
    _need_tiled(x_q, m, k, "x_q")
    _need_tiled(w_q, n, k, "w_q")
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_w8a8_gemm_per_tensor_tiled", _ptr(x_q), _ptr(x_scale), m, _ptr(w_q), _ptr(w_scale), n, k,
                   _ptr(bias), bt, _ptr(y), _dtype_code(y), _stream(stream, y))


def sq_wo_linear(x: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor, bias: torch.Tensor | None,
                 y: torch.Tensor, stream=None) -> int:
    """Weight-only int8 linear: y = (x @ w_q^T) * w_scale + bias, x bf16."""
    m, k = x.shape
    n = w_q.shape[0]
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_wo_linear", _ptr(x), _dtype_code(x), m, k, _ptr(w_q), _ptr(w_scale), n, _ptr(bias), bt,
                   _ptr(y), _dtype_code(y), _stream(stream, x))


def sq_wo_linear_tiled(x: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor, n: int,
                       bias: torch.Tensor | None, y: torch.Tensor, stream=None) -> int:
    """sq_wo_linear with w_q (flat int8) in 16 x 64 tiles."""
    m, k = x.shape
    _need_tiled(w_q, n, k, "w_q")
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_wo_linear_tiled", _ptr(x), _dtype_code(x), m, k, _ptr(w_q), _ptr(w_scale), n, _ptr(bias),
                   bt, _ptr(y), _dtype_code(y), _stream(stream, x))


def sq_weight_col_max(w: torch.Tensor, w_max_abs: torch.Tensor, stream=None) -> int:
    """w_max_abs[j] = max(max_o |w[o, j]|, 1e-8)."""
    n, k = w.shape
    _need_dtype(w_max_abs, torch.float32, "w_max_abs")
    return _invoke("sq_weight_col_max", _ptr(w), _dtype_code(w), n, k, _ptr(w_max_abs), _stream(stream, w))


def sq_recompute_smooth_scale(w: torch.Tensor, x_max_abs: torch.Tensor | None, w_max_abs: torch.Tensor | None,
                              alpha: float, smooth: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                              stream=None) -> int:
    """s, int8 weights and scales for a new alpha from the stored maxima (one
    pass over w); SQ_WARN_UNCALIBRATED when x_max_abs is None."""
    n, k = w.shape
    _need_dtype(smooth, torch.float32, "smooth")
    _need_dtype(w_q, torch.int8, "w_q")
    _need_dtype(w_scale, torch.float32, "w_scale")
    for t, nm in ((x_max_abs, "x_max_abs"), (w_max_abs, "w_max_abs")):
        if t is not None:
            _need_dtype(t, torch.float32, nm)
    return _invoke("sq_recompute_smooth_scale", _ptr(w), _dtype_code(w), n, k, _ptr(x_max_abs), _ptr(w_max_abs),
                   float(alpha), _ptr(smooth), _ptr(w_q), _ptr(w_scale), _stream(stream, w))


def sq_tiled_bytes(rows: int, k: int) -> int:
    """Bytes of a [rows][k] int8 matrix in 16 x 64 tiles."""
    return int(lib().sq_tiled_bytes(rows, k))


def tiled_empty(rows: int, k: int, device) -> torch.Tensor:
    """A flat int8 device buffer for a [rows][k] matrix in 16 x 64 tiles."""
    return torch.empty(max(sq_tiled_bytes(rows, k), 16), dtype=torch.int8, device=device)


def _need_tiled(t: torch.Tensor, rows: int, k: int, what: str):
    _need_dtype(t, torch.int8, what)
    if t.numel() < sq_tiled_bytes(rows, k):
        raise ValueError(f"{what} needs {sq_tiled_bytes(rows, k)} bytes for {rows} x {k} in tiles")


def sq_prepare_weight_tiled(w: torch.Tensor, x_max_abs: torch.Tensor | None, alpha: float, smooth: torch.Tensor,
                            w_q: torch.Tensor, w_scale: torch.Tensor, stream=None) -> int:
    """sq_prepare_weight with w_q (flat int8) in 16 x 64 tiles."""
    n, k = w.shape
    _need_dtype(smooth, torch.float32, "smooth")
    _need_tiled(w_q, n, k, "w_q")
    _need_dtype(w_scale, torch.float32, "w_scale")
    if x_max_abs is not None:
        _need_dtype(x_max_abs, torch.float32, "x_max_abs")
    return _invoke("sq_prepare_weight_tiled", _ptr(w), _dtype_code(w), n, k, _ptr(x_max_abs), float(alpha),
                   _ptr(smooth), _ptr(w_q), _ptr(w_scale), _stream(stream, w))


def sq_quantize_act_tiled(x: torch.Tensor, smooth: torch.Tensor, x_q: torch.Tensor, x_scale: torch.Tensor,
                          stream=None) -> int:
    """sq_quantize_act with x_q (flat int8) in 16 x 64 tiles."""
    m, k = x.shape
    _need_tiled(x_q, m, k, "x_q")
    _need_dtype(x_scale, torch.float32, "x_scale")
    return _invoke("sq_quantize_act_tiled", _ptr(x), _dtype_code(x), m, k, _ptr(smooth), _ptr(x_q), _ptr(x_scale),
                   _stream(stream, x))


def sq_w8a8_gemm_tiled(x_q: torch.Tensor, x_scale: torch.Tensor | None, m: int, w_q: torch.Tensor,
                       w_scale: torch.Tensor | None, n: int, k: int, bias: torch.Tensor | None, y: torch.Tensor,
                       stream=None) -> int:
    """sq_w8a8_gemm on operands in 16 x 64 tiles (flat int8 buffers; the
    shape is given)."""
    _need_tiled(x_q, m, k, "x_q")
    _need_tiled(w_q, n, k, "w_q")
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_w8a8_gemm_tiled", _ptr(x_q), _ptr(x_scale), m, _ptr(w_q), _ptr(w_scale), n, k, _ptr(bias), bt,
                   _ptr(y), _dtype_code(y), _stream(stream, y))


def untile(t: torch.Tensor, rows: int, k: int) -> torch.Tensor:
    """The [rows][k] matrix held by a 16 x 64 tiled buffer (host-side view
    helper for tests and inspection; a copy)."""
    r16, k64 = (rows + 15) // 16 * 16, (k + 63) // 64 * 64
    a = t[: r16 * k64].reshape(r16 // 16, k64 // 64, 16, 64).permute(0, 2, 1, 3).reshape(r16, k64)
    return a[:rows, :k].contiguous()


def sq_smoothing_factor(x_max_abs: torch.Tensor | None, w_max_abs: torch.Tensor, alpha: float, smooth: torch.Tensor,
                        stream=None) -> int:
    """s from the stored maxima (SQ_WARN_UNCALIBRATED when x_max_abs is None)."""
    k = smooth.numel()
    for t, nm in ((x_max_abs, "x_max_abs"), (w_max_abs, "w_max_abs"), (smooth, "smooth")):
        if t is not None:
            _need_dtype(t, torch.float32, nm)
            if t.numel() != k:
                raise ValueError(f"{nm} must have {k} elements")
    return _invoke("sq_smoothing_factor", _ptr(x_max_abs), _ptr(w_max_abs), float(alpha), k, _ptr(smooth),
                   _stream(stream, smooth))


def sq_quantize_weight(w: torch.Tensor, smooth: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                       stream=None) -> int:
    """Int8 codes and per-output-channel scales of w * smooth."""
    n, k = w.shape
    _need_dtype(smooth, torch.float32, "smooth")
    _need_dtype(w_q, torch.int8, "w_q")
    _need_dtype(w_scale, torch.float32, "w_scale")
    return _invoke("sq_quantize_weight", _ptr(w), _dtype_code(w), n, k, _ptr(smooth), _ptr(w_q), _ptr(w_scale),
                   _stream(stream, w))


def sq_reference_linear(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None, y: torch.Tensor,
                        stream=None) -> int:
    """The unquantised linear y = x w^T + bias (x and w both fp32 or both
    bf16; fp32 sums)."""
    m, k = x.shape
    n = w.shape[0]
    if w.dtype != x.dtype or w.shape[1] != k:
        raise TypeError("w must have x's dtype and k columns")
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    return _invoke("sq_reference_linear", _ptr(x), _dtype_code(x), m, k, _ptr(w), n, _ptr(bias), bt, _ptr(y),
                   _dtype_code(y), _stream(stream, x))


def sq_relative_error_workspace_bytes(count: int) -> int:
    return int(lib().sq_relative_error_workspace_bytes(count))


def sq_relative_error(y_fp: torch.Tensor, y_q: torch.Tensor, workspace: torch.Tensor, result: torch.Tensor,
                      stream=None) -> int:
    """result (3 float64, device) = ||y_fp - y_q||_F, ||y_fp||_F and their
    ratio (denominator floored at 1e-12); y_fp and y_q fp32 of one size."""
    _need_dtype(y_fp, torch.float32, "y_fp")
    _need_dtype(y_q, torch.float32, "y_q")
    _need_dtype(result, torch.float64, "result")
    if y_fp.numel() != y_q.numel() or result.numel() < 3:
        raise ValueError("y_fp and y_q must have one size, result at least 3 elements")
    nbytes = workspace.numel() * workspace.element_size()
    return _invoke("sq_relative_error", _ptr(y_fp), _ptr(y_q), y_fp.numel(), _ptr(workspace), nbytes,
                   _ptr(result), _stream(stream, y_fp))


def sq_selfcheck_reciprocal(mismatches: torch.Tensor, stream=None) -> int:
    """Adds to mismatches[0] (int64, device) the count of s in [2^-100, 2^100)
    whose kernel reciprocal differs from the IEEE 1/s."""
    _need_dtype(mismatches, torch.int64, "mismatches")
    return _invoke("sq_selfcheck_reciprocal", _ptr(mismatches), _stream(stream, mismatches))


def sq_selfcheck_division(b_begin: int, b_end: int, mismatches: torch.Tensor, stream=None) -> int:
    """Adds to mismatches[0] (int64, device) the count of significand pairs
    (divisors [b_begin, b_end)) whose kernel quotient differs from IEEE a/b."""
    _need_dtype(mismatches, torch.int64, "mismatches")
    return _invoke("sq_selfcheck_division", b_begin, b_end, _ptr(mismatches), _stream(stream, mismatches))


def sq_w8a8_linear_workspace_bytes(m: int, k: int) -> int:
    return lib().sq_w8a8_linear_workspace_bytes(m, k)


def workspace_views(workspace: torch.Tensor, m: int, k: int):
    """(x_q [m, k] int8, x_scale [m] fp32) views of a linear's workspace."""
    off = (m * k + 255) // 256 * 256
    xq = workspace[: m * k].view(torch.int8).view(m, k)
    xs = workspace[off: off + 4 * m].view(torch.float32)
    return xq, xs


def sq_w8a8_linear(x: torch.Tensor, smooth: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                   bias: torch.Tensor | None, y: torch.Tensor, workspace: torch.Tensor, stream=None) -> int:
    """One frozen forward (activation quantisation + int8 GEMM + dequant)."""
    m, k = x.shape
    n = w_q.shape[0]
    if bias is not None:
        _need_dtype(bias, x.dtype, "bias")
    nbytes = workspace.numel() * workspace.element_size()
    return _invoke("sq_w8a8_linear", _ptr(x), _dtype_code(x), m, k, _ptr(smooth), _ptr(w_q), _ptr(w_scale), n,
                   _ptr(bias), _ptr(y), _dtype_code(y), _ptr(workspace), nbytes, _stream(stream, x))


def sq_w8a8_linear_tiled_workspace_bytes(m: int, k: int) -> int:
    return int(lib().sq_w8a8_linear_tiled_workspace_bytes(m, k))


def sq_w8a8_linear_tiled_fused_workspace_bytes(m: int, k: int) -> int:
    return int(lib().sq_w8a8_linear_tiled_fused_workspace_bytes(m, k))


def linear_tiled_workspace(m: int, k: int, device, fused: bool = False) -> torch.Tensor:
    """A workspace for sq_w8a8_linear_tiled, or zero-filled for
    sq_w8a8_linear_tiled_fused (the zeros are the initial state of its
    synchronisation words)."""
    nbytes = (sq_w8a8_linear_tiled_fused_workspace_bytes if fused else sq_w8a8_linear_tiled_workspace_bytes)(m, k)
    return torch.zeros(max(nbytes, 1024 if fused else 256), dtype=torch.uint8, device=device)


def linear_tiled_views(workspace: torch.Tensor, m: int, k: int, fused: bool = False):
    """(x_q in tiles (flat int8), x_scale [m] fp32) views of a
    sq_w8a8_linear_tiled(_fused) workspace."""
    base = 1024 if fused else 0
    tb = sq_tiled_bytes(m, k)
    off = base + (tb + 255) // 256 * 256
    return workspace[base: base + tb].view(torch.int8), workspace[off: off + 4 * m].view(torch.float32)


def linear_tiled_fallbacks(workspace: torch.Tensor) -> int:
    """How many workgroups of sq_w8a8_linear_tiled_fused have run out of
    polls and quantised the tokens themselves, over every call on this
    workspace (a statistic the synchronisation words keep)."""
    return int(workspace[16:24].view(torch.int64).item())


def sq_w8a8_linear_tiled(x: torch.Tensor, smooth: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor, n: int,
                         bias: torch.Tensor | None, y: torch.Tensor, workspace: torch.Tensor, stream=None) -> int:
    """One forward on tiled int8 weights (activation codes into the
    workspace, then the product)."""
    m, k = x.shape
    _need_tiled(w_q, n, k, "w_q")
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    nbytes = workspace.numel() * workspace.element_size()
    return _invoke("sq_w8a8_linear_tiled", _ptr(x), _dtype_code(x), m, k, _ptr(smooth), _ptr(w_q), _ptr(w_scale), n,
                   _ptr(bias), bt, _ptr(y), _dtype_code(y), _ptr(workspace), nbytes, _stream(stream, x))


def sq_w8a8_linear_tiled_fused(x: torch.Tensor, smooth: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                               n: int, bias: torch.Tensor | None, y: torch.Tensor, workspace: torch.Tensor,
                               stream=None) -> int:
    """The same forward as one kernel (up to 64 tokens); the workspace
    (linear_tiled_workspace(..., fused=True)) must have been zero-filled once."""
    m, k = x.shape
    _need_tiled(w_q, n, k, "w_q")
    bt = _dtype_code(bias) if bias is not None else SQ_F32
    nbytes = workspace.numel() * workspace.element_size()
    return _invoke("sq_w8a8_linear_tiled_fused", _ptr(x), _dtype_code(x), m, k, _ptr(smooth), _ptr(w_q),
                   _ptr(w_scale), n, _ptr(bias), bt, _ptr(y), _dtype_code(y), _ptr(workspace), nbytes,
                   _stream(stream, x))


def sq_set_fused_wait_polls(polls: int) -> None:
    lib().sq_set_fused_wait_polls(int(polls))


def sq_w8a8_linear_noalloc(x: torch.Tensor, smooth: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor,
                           bias: torch.Tensor | None, y: torch.Tensor, stream=None) -> int:
    """sq_w8a8_linear with the activation codes in the library's own fixed
    device array (no workspace, nothing allocated; calls overlapping on one
    GPU race)."""
    m, k = x.shape
    n = w_q.shape[0]
    if bias is not None:
        _need_dtype(bias, x.dtype, "bias")
    return _invoke("sq_w8a8_linear_noalloc", _ptr(x), _dtype_code(x), m, k, _ptr(smooth), _ptr(w_q),
                   _ptr(w_scale), n, _ptr(bias), _ptr(y), _dtype_code(y), _stream(stream, x))


def sq_alpha_from_eta(eta: float) -> float:
    """alpha = sigmoid(eta) (binary64, rounded to binary32)."""
    return float(lib().sq_alpha_from_eta(float(eta)))


def sq_eta_from_alpha(alpha: float) -> float:
    """The page's initial eta for an initial alpha: log(a / max(1e-6, 1 - a))."""
    return float(lib().sq_eta_from_alpha(float(alpha)))


def sq_ste_backward_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().sq_ste_backward_workspace_bytes(m, n, k))


def sq_ste_backward(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, smooth: torch.Tensor, x_q: torch.Tensor,
                    x_scale: torch.Tensor, w_q: torch.Tensor, w_scale: torch.Tensor, x_max_abs: torch.Tensor | None,
                    w_max_abs: torch.Tensor | None, alpha: float, dx: torch.Tensor, dw: torch.Tensor,
                    dbias: torch.Tensor | None, dsmooth: torch.Tensor | None, dalpha_deta: torch.Tensor,
                    workspace: torch.Tensor, stream=None) -> int:
    """The straight-through backward: dx, dw, dbias, dsmooth and
    (dalpha, deta) for the upstream gradient dy (SQ_WARN_UNCALIBRATED when
    x_max_abs is None: no alpha gradient)."""
    m, n = dy.shape
    k = x.shape[1]
    for t, nm in ((dx, "dx"), (dw, "dw"), (smooth, "smooth"), (x_scale, "x_scale"), (w_scale, "w_scale")):
        _need_dtype(t, torch.float32, nm)
    for t, nm in ((dbias, "dbias"), (dsmooth, "dsmooth"), (x_max_abs, "x_max_abs"), (w_max_abs, "w_max_abs")):
        if t is not None:
            _need_dtype(t, torch.float32, nm)
    _need_dtype(dalpha_deta, torch.float64, "dalpha_deta")
    if x.shape != (m, k) or w.shape != (n, k) or x_q.shape != (m, k) or w_q.shape != (n, k):
        raise ValueError("x [m][k], w [n][k] and their codes must match dy [m][n]")
    nbytes = workspace.numel() * workspace.element_size()
    return _invoke("sq_ste_backward", _ptr(dy), _dtype_code(dy), m, n, k, _ptr(x), _dtype_code(x), _ptr(w),
                   _dtype_code(w), _ptr(smooth), _ptr(x_q), _ptr(x_scale), _ptr(w_q), _ptr(w_scale),
                   _ptr(x_max_abs), _ptr(w_max_abs), float(alpha), _ptr(dx), _ptr(dw), _ptr(dbias), _ptr(dsmooth),
                   _ptr(dalpha_deta), _ptr(workspace), nbytes, _stream(stream, dy))


def sq_aux_loss_grad_workspace_bytes(count: int) -> int:
    return int(lib().sq_aux_loss_grad_workspace_bytes(count))


def sq_aux_loss_grad(y_fp: torch.Tensor, y_q: torch.Tensor, dy_q: torch.Tensor, loss: torch.Tensor,
                     workspace: torch.Tensor, stream=None) -> int:
    """loss = ||y_fp - y_q||^2 / ||y_fp||^2 (binary64, device) and its
    gradient at y_q (fp32)."""
    for t, nm in ((y_fp, "y_fp"), (y_q, "y_q"), (dy_q, "dy_q")):
        _need_dtype(t, torch.float32, nm)
    _need_dtype(loss, torch.float64, "loss")
    if y_fp.numel() != y_q.numel() or dy_q.numel() != y_q.numel():
        raise ValueError("y_fp, y_q and dy_q must have one size")
    nbytes = workspace.numel() * workspace.element_size()
    return _invoke("sq_aux_loss_grad", _ptr(y_fp), _ptr(y_q), y_q.numel(), _ptr(dy_q), _ptr(loss), _ptr(workspace),
                   nbytes, _stream(stream, y_q))


# ---------------------------------------------------------------------------
# The page's layer lifecycle on top of the ABI: calibrate -> freeze -> forward
# (SmoothQuantW8A8 in "w8a8_smoothquant.py"). Buffers only; no arithmetic.
# ---------------------------------------------------------------------------
class SmoothQuantLinear:
    """Holds a layer's buffers and drives the ABI in the page's order.

    layout "row" keeps the int8 weights as [n][k] row-major and runs the
    forward as one sq_w8a8_linear call (sq_quantize_act + sq_w8a8_gemm when
    the bias type differs from x's); "tiled" keeps them in 16 x 64 tiles
    (flat, sq_tiled_bytes(n, k)) and runs the forward as one
    sq_w8a8_linear_tiled call. Both give the same smoothing
    factor, scales, codes and outputs, bit for bit; the tiled products are
    the faster ones."""

    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None, alpha: float = 0.5,
                 layout: str = "row", learnable_alpha: bool = False):
        if not weight.is_cuda:
            raise ValueError("weight must be a device tensor")
        if layout not in ("row", "tiled"):
            raise ValueError(f"layout must be 'row' or 'tiled', not {layout!r}")
        self.layout = layout
        self.weight = weight.contiguous()
        self.bias = None if bias is None else bias.contiguous()
        self.alpha = float(alpha)
        n, k = self.weight.shape
        dev = self.weight.device
        self.calib_max_abs = torch.zeros(k, dtype=torch.float32, device=dev)
        self.calib_count = 0
        self.smooth = torch.ones(k, dtype=torch.float32, device=dev)
        if layout == "tiled":
            self.weight_int8 = tiled_empty(n, k, dev).zero_()
        else:
            self.weight_int8 = torch.zeros((n, k), dtype=torch.int8, device=dev)
        self.weight_scale = torch.ones(n, dtype=torch.float32, device=dev)
        self.weight_max_abs = torch.empty(k, dtype=torch.float32, device=dev)
        self.is_quantized = False
        # the page's learnable alpha: alpha = sigmoid(eta), eta initialised
        # from the given alpha (then alpha is eta's sigmoid, not exactly it)
        self.learnable_alpha = bool(learnable_alpha)
        self.eta = sq_eta_from_alpha(alpha) if learnable_alpha else None
        if learnable_alpha:
            self.alpha = sq_alpha_from_eta(self.eta)
        self._saved = None

    def calibrate(self, x: torch.Tensor) -> None:
        if self.is_quantized:
            raise RuntimeError("calibration after freeze is not allowed")
        x2 = x.reshape(-1, x.shape[-1])
        if self.calib_count == 0:
            sq_calibrate_first(x2, self.calib_max_abs)
        else:
            sq_calibrate(x2, self.calib_max_abs)
        self.calib_count += x2.shape[0]

    def calibrate_batches(self, xs) -> None:
        """Several device-resident calibration batches at once, up to
        SQ_MAX_CALIB_BATCHES per call of sq_calibrate_batches: the same running
        max as calibrate on each batch in turn."""
        if self.is_quantized:
            raise RuntimeError("calibration after freeze is not allowed")
        xs = [x.reshape(-1, x.shape[-1]) for x in xs]
        for i in range(0, len(xs), SQ_MAX_CALIB_BATCHES):
            chunk = xs[i:i + SQ_MAX_CALIB_BATCHES]
            sq_calibrate_batches(chunk, self.calib_max_abs, first=self.calib_count == 0)
            self.calib_count += sum(x.shape[0] for x in chunk)

    def freeze(self) -> int:
        """Returns SQ_OK, or SQ_WARN_UNCALIBRATED when no batch was seen. The
        weight column max is kept for recompute."""
        sq_weight_col_max(self.weight, self.weight_max_abs)
        st = self._quantize_weight()
        self.is_quantized = True
        return st

    def _quantize_weight(self) -> int:
        mx = self.calib_max_abs if self.calib_count else None
        if self.layout == "tiled":
            # the tiled weight preparation takes the weight column max itself
            # (one more pass over W than the route from the stored maxima)
            return sq_prepare_weight_tiled(self.weight, mx, self.alpha, self.smooth, self.weight_int8,
                                           self.weight_scale)
        return sq_recompute_smooth_scale(self.weight, mx, self.weight_max_abs, self.alpha, self.smooth,
                                         self.weight_int8, self.weight_scale)

    def recompute(self, alpha: float) -> int:
        """recompute_smooth_scale: re-smooth and re-quantise the weights for a
        new alpha from the stored maxima (one pass over the weights)."""
        if not self.is_quantized:
            raise RuntimeError("recompute before freeze")
        self.alpha = float(alpha)
        return self._quantize_weight()

    def set_eta(self, eta: float) -> int:
        """The learnable alpha's parameter: alpha = sigmoid(eta); the weights
        are re-smoothed and re-quantised for it (one pass over W)."""
        if not self.learnable_alpha:
            raise RuntimeError("alpha is not learnable for this layer")
        self.eta = float(eta)
        return self.recompute(sq_alpha_from_eta(self.eta))

    def train_forward(self, x: torch.Tensor) -> torch.Tensor:
        """The quantized forward in fp32 (as the page's training forward),
        keeping what the straight-through backward needs (row layout)."""
        if not self.is_quantized:
            raise RuntimeError("forward before freeze")
        if self.layout != "row":
            raise RuntimeError("the straight-through backward takes row-major codes (layout='row')")
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        m, k = x2.shape
        n = self.weight_scale.shape[0]
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
        x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
        sq_quantize_act(x2, self.smooth, x_q, x_scale)
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
        sq_w8a8_gemm(x_q, x_scale, self.weight_int8, self.weight_scale, self.bias, y)
        self._saved = (x2, x_q, x_scale, x.shape)
        return y.reshape(*x.shape[:-1], n)

    def backward(self, dy: torch.Tensor) -> dict:
        """The straight-through backward of the last train_forward for the
        upstream gradient dy: dict with dx, dw, dbias (None without a
        bias), dsmooth (device tensors), dalpha and deta (floats; zero when
        the layer was never calibrated)."""
        if self._saved is None:
            raise RuntimeError("backward before train_forward")
        x2, x_q, x_scale, xshape = self._saved
        m, k = x2.shape
        n = self.weight_scale.shape[0]
        dy2 = dy.reshape(m, n).contiguous()
        dev = x2.device
        dx = torch.empty((m, k), dtype=torch.float32, device=dev)
        dw = torch.empty((n, k), dtype=torch.float32, device=dev)
        db = torch.empty(n, dtype=torch.float32, device=dev) if self.bias is not None else None
        ds = torch.empty(k, dtype=torch.float32, device=dev)
        da = torch.empty(2, dtype=torch.float64, device=dev)
        ws = torch.empty(max(sq_ste_backward_workspace_bytes(m, n, k), 256), dtype=torch.uint8, device=dev)
        mx = self.calib_max_abs if self.calib_count else None
        sq_ste_backward(dy2, x2, self.weight, self.smooth, x_q, x_scale, self.weight_int8, self.weight_scale, mx,
                        self.weight_max_abs, self.alpha, dx, dw, db, ds, da, ws)
        dah = da.cpu()
        return dict(dx=dx.reshape(xshape), dw=dw, dbias=db, dsmooth=ds, dalpha=float(dah[0]), deta=float(dah[1]))

    def quantization_error(self, x: torch.Tensor) -> float:
        """||Y_fp - Y_q||_F / max(||Y_fp||_F, 1e-12): the unquantised linear
        against the quantized forward, both fp32 outputs."""
        if not self.is_quantized:
            raise RuntimeError("quantization_error before freeze")
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        w = self.weight
        xr = x2
        if w.dtype != x2.dtype:
            # the reference takes one operand type: widen the bf16 side to
            # fp32 (exact), never narrow the other
            xr, w = x2.float(), w.float()
        y_fp = torch.empty((x2.shape[0], w.shape[0]), dtype=torch.float32, device=x2.device)
        sq_reference_linear(xr, w, self.bias, y_fp)
        y_q = self.forward(x2, out_dtype=torch.float32)
        ws = torch.empty(max(sq_relative_error_workspace_bytes(y_fp.numel()), 8), dtype=torch.uint8,
                         device=x2.device)
        result = torch.empty(3, dtype=torch.float64, device=x2.device)
        sq_relative_error(y_fp, y_q, ws, result)
        return float(result[2].item())

    def forward(self, x: torch.Tensor, out_dtype: torch.dtype | None = None) -> torch.Tensor:
        if not self.is_quantized:
            raise RuntimeError("forward before freeze")
        shape = x.shape
        x2 = x.reshape(-1, shape[-1]).contiguous()
        m, k = x2.shape
        n = self.weight_scale.shape[0]
        y = torch.empty((m, n), dtype=out_dtype or x.dtype, device=x.device)
        if self.layout == "tiled":
            if m:
                ws = torch.empty(sq_w8a8_linear_tiled_workspace_bytes(m, k), dtype=torch.uint8, device=x.device)
                sq_w8a8_linear_tiled(x2, self.smooth, self.weight_int8, self.weight_scale, n, self.bias, y, ws)
        elif self.bias is not None and self.bias.dtype != x2.dtype:
            # sq_w8a8_linear takes the bias in x's type; another bias type
            # goes through the two calls it is made of, which take its type
            if m:
                x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
                x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
                sq_quantize_act(x2, self.smooth, x_q, x_scale)
                sq_w8a8_gemm(x_q, x_scale, self.weight_int8, self.weight_scale, self.bias, y)
        else:
            ws = torch.empty(max(sq_w8a8_linear_workspace_bytes(m, k), 1), dtype=torch.uint8, device=x.device)
            sq_w8a8_linear(x2, self.smooth, self.weight_int8, self.weight_scale, self.bias, y, ws)
        return y.reshape(*shape[:-1], n)
