"""CPU oracle for the SmoothQuant W8A8 quantized linear (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library under
``w8a8_quantized_linear_sq_amd``) never imports, links or calls it, and the two
share no code.

The arithmetic lives in ``sq_oracle.c`` (plain C99, gcc ``-O2
-ffp-contract=off``, no fast-math); this module builds it and marshals numpy
arrays into it. Every function follows the page "w8a8_smoothquant.py"
(BiGRU_T_version): see the docstring of each wrapper.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, exact rational brute force, a hand-derived worked example under
``tests/golden/``, invariants, and mutants of this very file that each pin set
must reject).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsq_oracle.so")

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-fopenmp", "-Wall", "-Wextra"]


# AddressSanitizer and UndefinedBehaviorSanitizer for a checked CPU build
# (the sanitizer runtimes must then be preloaded into the host process).
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(out_path: str = _LIB_PATH, mutant: int = 0, sanitize: bool = False) -> str:
    """Compile the oracle with gcc. ``mutant`` > 0 plants one deliberate
    mistake (the MUTANT sites in sq_oracle.c) for the pin-sensitivity tests;
    ``sanitize`` builds it with AddressSanitizer and UBSan."""
    flags = [f for f in CFLAGS if not (sanitize and f == "-fopenmp")]
    cmd = ["gcc", *flags, *(SANITIZE if sanitize else []), f"-DSQO_MUTANT={int(mutant)}", _SRC, "-o",
           out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    sig = {
        "sqo_mutant": ([], ctypes.c_int),
        "sqo_calibrate": ([_P, _I64, _I64, _P], None),
        "sqo_weight_col_max": ([_P, _I64, _I64, _P], None),
        "sqo_smoothing_factor": ([_P, _P, ctypes.c_float, _I64, _P], ctypes.c_int),
        "sqo_smooth_weight": ([_P, _P, _I64, _I64, _P], None),
        "sqo_smooth_act": ([_P, _P, _I64, _I64, _P], None),
        "sqo_quantize_rows": ([_P, _I64, _I64, _P, _P], None),
        "sqo_quantize_tensor": ([_P, _I64, _P, _P], None),
        "sqo_wo_linear": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], None),
        "sqo_int_gemm": ([_P, _P, _I64, _I64, _I64, _P], _I64),
        "sqo_dequant": ([_P, _P, _P, _P, _I64, _I64, _P], None),
        "sqo_simulated_forward": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], None),
        "sqo_f64_to_bf16": ([_P, _I64, _P], None),
        "sqo_reference_linear": ([_P, _P, _P, _I64, _I64, _I64, _P], None),
        "sqo_relative_error": ([_P, _P, _I64, _P], ctypes.c_double),
        "sqo_alpha_from_eta": ([ctypes.c_float], ctypes.c_float),
        "sqo_eta_from_alpha": ([ctypes.c_double], ctypes.c_float),
        "sqo_ste_backward": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I64, _I64, _I64,
                              _P, _P, _P, _P, _P, _P, _P], None),
        "sqo_ste_chain": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I64, _I64, _I64, _P, _P, _P, _P], None),
        "sqo_aux_loss_grad": ([_P, _P, _I64, _P], ctypes.c_double),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


class Oracle:
    """numpy front end of one build of sq_oracle.c."""

    def __init__(self, lib_path: str = _LIB_PATH):
        if not os.path.exists(lib_path) or (
                lib_path == _LIB_PATH and os.path.getmtime(_SRC) > os.path.getmtime(lib_path)):
            build(lib_path)
        self.lib = _bind(ctypes.CDLL(lib_path))
        self.mutant = self.lib.sqo_mutant()

    # -- helpers ----------------------------------------------------------
    @staticmethod
    def _f32(a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float32)
        return a

    @staticmethod
    def _ptr(a: np.ndarray | None):
        return None if a is None else a.ctypes.data

    # -- the page's steps ---------------------------------------------------
    def calibrate(self, x, running=None) -> np.ndarray:
        """SmoothQuantW8A8.calibrate: running per-channel max of |X| (no floor).
        ``running`` (float32[k]) is updated in place if given, else starts at 0."""
        x = self._f32(x)
        k = x.shape[-1]
        x2 = x.reshape(-1, k)
        if running is None:
            running = np.zeros(k, np.float32)
        assert running.dtype == np.float32 and running.flags.c_contiguous
        self.lib.sqo_calibrate(self._ptr(x2), x2.shape[0], k, self._ptr(running))
        return running

    def weight_col_max(self, w) -> np.ndarray:
        """calibrate_smoothquant's max_w: max over output rows of |W|, floored."""
        w = self._f32(w)
        n, k = w.shape
        mw = np.empty(k, np.float32)
        self.lib.sqo_weight_col_max(self._ptr(w), n, k, self._ptr(mw))
        return mw

    def smoothing_factor(self, mx, mw, alpha: float) -> np.ndarray:
        """calibrate_smoothquant: s = max(mx,1e-8)^a / mw^(1-a), floored at 1e-8.
        ``mx`` None means never calibrated: s = 1."""
        mw = self._f32(mw)
        k = mw.shape[0]
        s = np.empty(k, np.float32)
        mxa = None if mx is None else self._f32(mx)
        self.lib.sqo_smoothing_factor(self._ptr(mxa), self._ptr(mw), float(alpha), k, self._ptr(s))
        return s

    def smooth_weight(self, w, s) -> np.ndarray:
        """freeze_quantization: W * s (column j times s_j), binary32."""
        w = self._f32(w)
        s = self._f32(s)
        n, k = w.shape
        out = np.empty_like(w)
        self.lib.sqo_smooth_weight(self._ptr(w), self._ptr(s), n, k, self._ptr(out))
        return out

    def smooth_act(self, x, s) -> np.ndarray:
        """forward: X / s (column j divided by s_j), binary32."""
        x = self._f32(x)
        s = self._f32(s)
        m, k = x.shape
        out = np.empty_like(x)
        self.lib.sqo_smooth_act(self._ptr(x), self._ptr(s), m, k, self._ptr(out))
        return out

    def quantize_rows(self, v):
        """quantize_per_channel_symmetric / quantize_per_token_symmetric:
        returns (int8 codes, float32 scale per row)."""
        v = self._f32(v)
        r, k = v.shape
        q = np.empty((r, k), np.int8)
        sc = np.empty(r, np.float32)
        self.lib.sqo_quantize_rows(self._ptr(v), r, k, self._ptr(q), self._ptr(sc))
        return q, sc

    def quantize_tensor(self, v):
        """quantize_tensor of the page "quantized_linear.py" (8 bits): one
        scale for the whole array; returns (int8 codes of v's shape, the
        float32 scale)."""
        v = self._f32(v)
        q = np.empty(v.shape, np.int8)
        sc = np.empty(1, np.float32)
        self.lib.sqo_quantize_tensor(self._ptr(v), v.size, self._ptr(q), self._ptr(sc))
        return q, np.float32(sc[0])

    def linear_per_tensor(self, x, w, bias=None):
        """QuantizedLinear of the page "quantized_linear.py" on the integer
        route: per-tensor codes of x and w, the int32 product, then
        acc * sx * sw + bias in binary64. Returns (xq, sx, wq, sw, acc, y)."""
        xq, sx = self.quantize_tensor(x)
        wq, sw = self.quantize_tensor(w)
        acc = self.int_gemm(xq, wq)
        m, n = acc.shape
        y = self.dequant(acc, np.full(m, sx, np.float32), np.full(n, sw, np.float32), bias)
        return xq, sx, wq, sw, acc, y

    def wo_linear(self, x, wq, sw, bias=None) -> np.ndarray:
        """Weight-only int8 linear (torchao Int8WeightOnlyQuantizedLinearWeight):
        (x @ wq^T) * scale_w[o] + bias[o] in binary64; x float32 [m, k]."""
        x = self._f32(x)
        wq = np.ascontiguousarray(wq, np.int8)
        sw = self._f32(sw)
        m, k = x.shape
        n = wq.shape[0]
        b = None if bias is None else self._f32(bias)
        y = np.empty((m, n), np.float64)
        self.lib.sqo_wo_linear(self._ptr(x), self._ptr(wq), self._ptr(sw), self._ptr(b), m, n, k, self._ptr(y))
        return y

    def reference_linear(self, x, w, bias=None) -> np.ndarray:
        """quantization_error's Y_fp: the unquantised linear x @ w^T + bias
        in binary64 (x [m, k], w [n, k] float32)."""
        x = self._f32(x)
        w = self._f32(w)
        m, k = x.shape
        n = w.shape[0]
        assert w.shape[1] == k
        b = None if bias is None else self._f32(bias)
        y = np.empty((m, n), np.float64)
        self.lib.sqo_reference_linear(self._ptr(x), self._ptr(w), self._ptr(b), m, n, k, self._ptr(y))
        return y

    def relative_error(self, y_fp, y_q):
        """quantization_error's measure ||y_fp - y_q||_F / max(||y_fp||_F,
        1e-12) in binary64; returns (ratio, ||y_fp - y_q||_F, ||y_fp||_F)."""
        a = np.ascontiguousarray(y_fp, np.float64)
        b = np.ascontiguousarray(y_q, np.float64)
        assert a.shape == b.shape
        norms = np.empty(2, np.float64)
        r = self.lib.sqo_relative_error(self._ptr(a), self._ptr(b), a.size, self._ptr(norms))
        return float(r), float(norms[0]), float(norms[1])

    def int_gemm(self, xq, wq) -> np.ndarray:
        """INT8 x INT8 -> INT32: acc[t, o] = sum_j xq[t, j] wq[o, j]."""
        xq = np.ascontiguousarray(xq, np.int8)
        wq = np.ascontiguousarray(wq, np.int8)
        m, k = xq.shape
        n, k2 = wq.shape
        assert k == k2
        acc = np.empty((m, n), np.int32)
        ov = self.lib.sqo_int_gemm(self._ptr(xq), self._ptr(wq), m, n, k, self._ptr(acc))
        if ov:
            raise OverflowError(f"{ov} accumulators exceed int32")
        return acc

    def dequant(self, acc, sx, sw, bias=None) -> np.ndarray:
        """acc * scale_x[t] * scale_w[o] + bias[o], binary64."""
        acc = np.ascontiguousarray(acc, np.int32)
        m, n = acc.shape
        sx = self._f32(sx)
        sw = self._f32(sw)
        b = None if bias is None else self._f32(bias)
        y = np.empty((m, n), np.float64)
        self.lib.sqo_dequant(self._ptr(acc), self._ptr(sx), self._ptr(sw), self._ptr(b), m, n,
                             self._ptr(y))
        return y

    def simulated_forward(self, xq, sx, wq, sw, bias=None) -> np.ndarray:
        """The page's fake-quant route: (xq*sx) @ (wq*sw)^T + bias in binary64."""
        xq = np.ascontiguousarray(xq, np.int8)
        wq = np.ascontiguousarray(wq, np.int8)
        m, k = xq.shape
        n = wq.shape[0]
        sx = self._f32(sx)
        sw = self._f32(sw)
        b = None if bias is None else self._f32(bias)
        y = np.empty((m, n), np.float64)
        self.lib.sqo_simulated_forward(self._ptr(xq), self._ptr(sx), self._ptr(wq), self._ptr(sw),
                                       self._ptr(b), m, n, k, self._ptr(y))
        return y

    def to_bf16(self, y) -> np.ndarray:
        """Round binary64 values once (nearest-even) to bf16; returns uint16 bits."""
        y = np.ascontiguousarray(y, np.float64)
        out = np.empty(y.shape, np.uint16)
        self.lib.sqo_f64_to_bf16(self._ptr(y), y.size, self._ptr(out))
        return out

    # -- the learnable alpha and the straight-through backward ---------------
    def alpha_from_eta(self, eta: float) -> np.float32:
        """SmoothQuantW8A8.alpha: sigmoid(eta) in binary64, rounded to binary32."""
        return np.float32(self.lib.sqo_alpha_from_eta(float(np.float32(eta))))

    def eta_from_alpha(self, alpha: float) -> np.float32:
        """SmoothQuantW8A8.__init__: log(a / max(1e-6, 1 - a)) stored as binary32."""
        return np.float32(self.lib.sqo_eta_from_alpha(float(alpha)))

    def ste_backward(self, dy, x, w, s, xq, sx, wq, sw, mx, mw, alpha):
        """The straight-through backward of the quantized forward (binary64):
        returns dict(gx, gw, dx, dw, db, ds, dalpha, deta); ``mx`` None =
        never calibrated (no alpha gradient)."""
        dy, x, w, s = self._f32(dy), self._f32(x), self._f32(w), self._f32(s)
        xq = np.ascontiguousarray(xq, np.int8)
        wq = np.ascontiguousarray(wq, np.int8)
        sx, sw, mw = self._f32(sx), self._f32(sw), self._f32(mw)
        mx = None if mx is None else self._f32(mx)
        m, k = x.shape
        n = w.shape[0]
        assert dy.shape == (m, n) and w.shape == (n, k) and xq.shape == (m, k) and wq.shape == (n, k)
        gx = np.empty((m, k), np.float64)
        gw = np.empty((n, k), np.float64)
        dx = np.empty((m, k), np.float64)
        dw = np.empty((n, k), np.float64)
        db = np.empty(n, np.float64)
        ds = np.empty(k, np.float64)
        da = np.empty(2, np.float64)
        self.lib.sqo_ste_backward(self._ptr(dy), self._ptr(x), self._ptr(w), self._ptr(s), self._ptr(xq),
                                  self._ptr(sx), self._ptr(wq), self._ptr(sw), self._ptr(mx), self._ptr(mw),
                                  float(np.float32(alpha)), m, n, k, self._ptr(gx), self._ptr(gw), self._ptr(dx),
                                  self._ptr(dw), self._ptr(db), self._ptr(ds), self._ptr(da))
        return dict(gx=gx, gw=gw, dx=dx, dw=dw, db=db, ds=ds, dalpha=float(da[0]), deta=float(da[1]))

    def ste_chain(self, gx, gw, x, w, s, mx, mw, alpha):
        """The chain rule from the gradients at X~ and W~ (binary64 arrays)
        to X, W, s, alpha and eta: returns dict(dx, dw, ds, dalpha, deta)."""
        gx = np.ascontiguousarray(gx, np.float64)
        gw = np.ascontiguousarray(gw, np.float64)
        x, w, s, mw = self._f32(x), self._f32(w), self._f32(s), self._f32(mw)
        mx = None if mx is None else self._f32(mx)
        m, k = x.shape
        n = w.shape[0]
        assert gx.shape == (m, k) and gw.shape == (n, k)
        dx = np.empty((m, k), np.float64)
        dw = np.empty((n, k), np.float64)
        ds = np.empty(k, np.float64)
        da = np.empty(2, np.float64)
        self.lib.sqo_ste_chain(self._ptr(gx), self._ptr(gw), self._ptr(x), self._ptr(w), self._ptr(s),
                               self._ptr(mx), self._ptr(mw), float(np.float32(alpha)), m, n, k, self._ptr(dx),
                               self._ptr(dw), self._ptr(ds), self._ptr(da))
        return dict(dx=dx, dw=dw, ds=ds, dalpha=float(da[0]), deta=float(da[1]))

    def aux_loss_grad(self, y_fp, y_q):
        """The docstring's auxiliary loss ||y_fp - y_q||^2 / ||y_fp||^2 and its
        gradient at y_q (binary64): returns (loss, dL/dy_q)."""
        a = np.ascontiguousarray(y_fp, np.float64)
        b = np.ascontiguousarray(y_q, np.float64)
        assert a.shape == b.shape
        g = np.empty(a.shape, np.float64)
        loss = self.lib.sqo_aux_loss_grad(self._ptr(a), self._ptr(b), a.size, self._ptr(g))
        return float(loss), g

    def training_step(self, x, w, bias, mx, eta, dy):
        """The quantized forward at alpha = sigmoid(eta) and its
        straight-through backward for the upstream gradient dy: returns the
        forward's quantities and the gradients (all from the oracle)."""
        alpha = self.alpha_from_eta(eta)
        mw = self.weight_col_max(w)
        s = self.smoothing_factor(mx, mw, alpha)
        wq, sw = self.quantize_rows(self.smooth_weight(w, s))
        xq, sx, acc, y = self.linear(x, s, wq, sw, bias)
        g = self.ste_backward(dy, x, w, s, xq, sx, wq, sw, mx, mw, alpha)
        return dict(alpha=alpha, mw=mw, s=s, wq=wq, sw=sw, xq=xq, sx=sx, y=y, **g)

    # -- compositions ---------------------------------------------------------
    def prepare_weight(self, w, mx, alpha: float):
        """freeze_quantization: (s, wq, scale_w) from the running max ``mx``
        (None = never calibrated)."""
        mw = self.weight_col_max(w)
        s = self.smoothing_factor(mx, mw, alpha)
        wq, sw = self.quantize_rows(self.smooth_weight(w, s))
        return s, wq, sw

    def quantize_act(self, x, s):
        """forward's activation side: per-token int8 of X / s."""
        return self.quantize_rows(self.smooth_act(x, s))

    def linear(self, x, s, wq, sw, bias=None):
        """forward, quantized branch: returns (xq, sx, acc int32, y binary64)."""
        xq, sx = self.quantize_act(x, s)
        acc = self.int_gemm(xq, wq)
        y = self.dequant(acc, sx, sw, bias)
        return xq, sx, acc, y


    def quantization_error(self, x, w, bias, mx, alpha: float) -> float:
        """SmoothQuantW8A8.quantization_error after a freeze with running max
        ``mx`` (None = never calibrated) and ``alpha``: the unquantised
        linear against the quantized forward (integer route), both binary64."""
        s, wq, sw = self.prepare_weight(w, mx, alpha)
        y_q = self.linear(x, s, wq, sw, bias)[3]
        return self.relative_error(self.reference_linear(x, w, bias), y_q)[0]


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from the unmodified source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def mutant(n: int, workdir: str | None = None) -> Oracle:
    """An oracle with deliberate mistake number ``n`` planted (tests only)."""
    d = workdir or tempfile.mkdtemp(prefix="sqo_mutant_")
    path = os.path.join(d, f"libsq_oracle_m{n}.so")
    build(path, mutant=n)
    return Oracle(path)
