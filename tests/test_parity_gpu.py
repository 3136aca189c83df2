"""GPU parity: every step of the HIP path against the CPU oracle, through the
C ABI, on seeded inputs. Bit-exact for maxima, s, scales, int8 codes and
int32 accumulators; fp32 outputs within 1e-6 of |acc sx sw| + |bias|; bf16
outputs within 1 bf16 ulp of the oracle's binary64 result rounded once."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from gpu_util import (DEV, assert_bf16_within_one_ulp, assert_equal, assert_f32_rel, down,
                      require_gpu, up)
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import inputs

pytestmark = pytest.mark.gpu

# (m, n, k): single elements, ragged tails of every tile, K tails of 16/32/48,
# several tiles, the largest K accepted (16384).
SMALL = [(1, 1, 16), (3, 5, 32), (7, 17, 48), (17, 33, 272), (33, 7, 16), (130, 260, 528),
         (257, 300, 1040), (64, 512, 4096), (5, 40, 11008), (300, 129, 2064), (70, 33, 16384)]
ALPHAS = [0.0, 0.25, 0.5, 0.75, 1.0, 0.3, None]


def _id(s):
    return "x".join(map(str, s))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    B.lib()


def _case(shape, dtype, seed=7, bias=True):
    m, n, k = shape
    return inputs.small(m, n, k, seed=seed + m + 3 * n + k, dtype=dtype, bias=bias)


def upo(t):
    return None if t is None else up(t)


def _zeros(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device=DEV)


# ---------------------------------------------------------------------------
# a1: running column max of |X|
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_calibrate(orc, shape, dtype):
    c = _case(shape, dtype)
    x = up(c.x)
    run = _zeros(c.k, torch.float32)
    # three uneven batches, last one first
    m = c.m
    cuts = sorted({0, m, max(0, m // 3), max(0, (2 * m) // 3)})
    for a, b in reversed(list(zip(cuts[:-1], cuts[1:]))):
        B.sq_calibrate(x[a:b], run)
    B.sq_calibrate(x[:0], run)  # empty batch: no-op
    torch.cuda.synchronize()
    assert_equal(down(run), orc.calibrate(c.x.f32), "running max")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,k", [(1, 16), (128, 4096), (129, 272), (2048, 4096), (5000, 1040), (64, 16384)],
                         ids=lambda v: str(v))
def test_calibrate_first(orc, rows, k, dtype):
    """sq_calibrate_first starts the running max from its batch whatever the
    buffer held (here values larger than any |x|), through the one-launch
    path (one row group) and the fill-and-fold path (several); later
    batches fold as usual."""
    c = inputs.small(rows, 8, k, seed=rows + k, dtype=dtype, bias=False)
    x = up(c.x)
    run = torch.full((k,), 1e30, dtype=torch.float32, device=DEV)
    half = rows // 2
    B.sq_calibrate_first(x[half:], run)
    B.sq_calibrate(x[:half], run)
    torch.cuda.synchronize()
    assert_equal(down(run), orc.calibrate(c.x.f32), "running max")
    empty = torch.full((k,), 5.0, dtype=torch.float32, device=DEV)
    B.sq_calibrate_first(x[:0], empty)
    torch.cuda.synchronize()
    assert not down(empty).any()


# batches (row counts) per call: the bench's four of 128 tokens, ragged runs
# with empty batches, the one-launch limit (1024 rows in all) and just past
# it (row groups folded with atomics), and long runs (one row per load)
BATCHES = [([128, 128, 128, 128], 4096), ([1, 0, 37, 5, 200, 3, 0, 17], 272), ([1024], 1040),
           ([600, 425], 4096), ([3000, 0, 2000, 100], 1040), ([2, 70], 16384), ([1], 16), ([0, 0], 64)]


@pytest.mark.parametrize("first", [0, 1])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,k", BATCHES, ids=lambda v: "-".join(map(str, v)) if isinstance(v, list) else str(v))
def test_calibrate_batches(orc, rows, k, dtype, first):
    """sq_calibrate_batches: every batch (separate buffers) folded at once,
    into a buffer that already holds the max of earlier rows (first == 0),
    or starting from these batches alone whatever the buffer held
    (first == 1); bit-exact against the oracle's running max over the same
    rows."""
    total = sum(rows)
    c = inputs.small(total + 9, 8, k, seed=total + k + 11, dtype=dtype, bias=False)
    x = up(c.x)
    cuts = np.cumsum([0] + rows)
    batches = [x[a:b].clone() for a, b in zip(cuts[:-1], cuts[1:])]
    prior = c.x.f32[total:]  # 9 rows calibrated before the call
    if first:
        run = torch.full((k,), 1e30, dtype=torch.float32, device=DEV)
        want = orc.calibrate(c.x.f32[:total]) if total else np.zeros(k, np.float32)
    else:
        run = up(orc.calibrate(prior))
        want = orc.calibrate(c.x.f32)
    torch.cuda.synchronize()
    B.sq_calibrate_batches(batches, run, first=bool(first))
    torch.cuda.synchronize()
    assert_equal(down(run), want, "running max")


# ---------------------------------------------------------------------------
# a2-a5: s, int8 weights, weight scales
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("alpha", ALPHAS, ids=lambda a: f"a{a}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL[::2] + [(64, 512, 4096)], ids=_id)
def test_prepare_weight(orc, shape, dtype, alpha):
    c = _case(shape, dtype)
    w = up(c.w)
    w_np = c.w.f32.copy()
    mx = orc.calibrate(c.x.f32)
    smooth = _zeros(c.k, torch.float32)
    wq = _zeros((c.n, c.k), torch.int8)
    ws = _zeros(c.n, torch.float32)
    st = B.sq_prepare_weight(w, None if alpha is None else up(mx), 0.5 if alpha is None else alpha,
                             smooth, wq, ws)
    torch.cuda.synchronize()
    assert st == (B.SQ_WARN_UNCALIBRATED if alpha is None else B.SQ_OK)
    s_gpu = down(smooth)
    s_ref = orc.smoothing_factor(None if alpha is None else mx, orc.weight_col_max(w_np),
                                 0.5 if alpha is None else alpha)
    if alpha in (None, 0.0, 0.25, 0.5, 0.75, 1.0):
        assert_equal(s_gpu, s_ref, "s")
    else:
        # alpha outside the exact forms: binary64 pow from two math libraries;
        # s may differ in the last bit, and everything after s must follow it
        ulps = np.abs(s_gpu.view(np.int32).astype(np.int64) - s_ref.view(np.int32))
        assert ulps.max() <= 1
    wq_ref, ws_ref = orc.quantize_rows(orc.smooth_weight(w_np, s_gpu))
    assert_equal(down(ws), ws_ref, "w_scale")
    assert_equal(down(wq), wq_ref, "w_q")


# ---------------------------------------------------------------------------
# a6-a7: per-token int8 of X / s
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_quantize_act(orc, shape, dtype):
    c = _case(shape, dtype)
    xf = c.x.f32.copy()
    if c.m > 2:
        xf[1] = 0.0  # an all-zero token: the floor decides its scale
    xt = inputs.Tensor(xf, None if c.x.bits is None else inputs.bf16_bits(xf))
    s, _, _ = orc.prepare_weight(c.w.f32, orc.calibrate(xf), 0.5)
    xq = _zeros((c.m, c.k), torch.int8)
    xs = _zeros(c.m, torch.float32)
    B.sq_quantize_act(up(xt), up(s), xq, xs)
    torch.cuda.synchronize()
    xq_ref, xs_ref = orc.quantize_act(xf, s)
    assert_equal(down(xs), xs_ref, "x_scale")
    assert_equal(down(xq), xq_ref, "x_q")


def _extreme_case(dtype, k=528, seed=3):
    """Activations and smoothing factors that reach every branch of the
    quotient x / s: quotients below 2^-50 (tiny x, or x over a huge s),
    subnormal x, quotients above 2^120 (huge x over a small s), factors at
    and above 2^40 (whose reciprocal is out of the fast path's range), zero
    rows, mixed rows. Every quotient and every row max stays finite."""
    rng = np.random.default_rng(seed)
    m = 12
    s = np.exp(rng.uniform(np.log(1e-8), np.log(1e4), size=k)).astype(np.float32)
    s[:8] = np.float32(2.0 ** 40)
    s[8:16] = np.float32(3.5e12)
    s[16:24] = np.float32(1e-8)
    x = (rng.standard_normal((m, k)) * 2.0).astype(np.float32)
    x[0] = (rng.standard_normal(k) * 1e-30).astype(np.float32)   # all quotients tiny
    x[1, ::3] = np.float32(1e-30)                                # tiny among normal
    x[2] = 0.0                                                   # zero row
    x[3, :] = 0.0
    x[3, 5] = np.float32(1e-41 if dtype == "f32" else 1e-39)     # subnormal, alone
    x[4, 24:40] = np.float32(2.5e36)                             # quotients above 2^120 where s >= 1
    x[5, :24] = np.float32(3e30)                                 # huge over huge or tiny s
    x[6, 16:24] = np.float32(1e30)                               # 1e30 / 1e-8 = 1e38: finite, above 2^120
    x[7, 8:16] = np.float32(-7.0)                                # normal over s >= 2^40
    x[8] = -x[8]
    # keep every quotient finite: rows with huge numerators only over s >= 1
    big = np.abs(x) > 1e29
    x[big & (s[None, :] < 1.0) & ~((np.arange(m)[:, None] == 6) & (np.arange(k)[None, :] < 24))] = 1.0
    if dtype == "bf16":
        bits = inputs.bf16_bits(x)
        return inputs.Tensor(inputs.bf16_to_f32(bits), bits), s
    return inputs.Tensor(x, None), s


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("shape", [(1024, 8208), (1030, 11008), (2051, 11264), (1000, 10000)], ids=_id)
def test_quantize_long_rows(orc, shape, tiled):
    """Rows of 8200-11264 channels: with 1024 rows or more the quantiser
    runs 384 threads x 4 chunks per row, below 1024 rows 704 x 2; both
    quantisers (activations and weights), both layouts, bit for bit."""
    r, k = shape
    c = inputs.small(r, r, k, seed=31 + r + k, dtype="bf16", bias=False)
    mx = orc.calibrate(c.x.f32)
    s, wq_ref, sw_ref = orc.prepare_weight(c.w.f32, mx, 0.5)
    xq_ref, xs_ref = orc.quantize_act(c.x.f32, s)
    xs, sw = _zeros(r, torch.float32), _zeros(r, torch.float32)
    s_dev = _zeros(k, torch.float32)
    if tiled:
        xq, wq = B.tiled_empty(r, k, DEV), B.tiled_empty(r, k, DEV)
        B.sq_quantize_act_tiled(up(c.x), up(s), xq, xs)
        B.sq_prepare_weight_tiled(up(c.w), up(mx), 0.5, s_dev, wq, sw)
        xq, wq = B.untile(xq, r, k), B.untile(wq, r, k)
    else:
        xq, wq = _zeros((r, k), torch.int8), _zeros((r, k), torch.int8)
        B.sq_quantize_act(up(c.x), up(s), xq, xs)
        B.sq_prepare_weight(up(c.w), up(mx), 0.5, s_dev, wq, sw)
    torch.cuda.synchronize()
    assert_equal(down(s_dev), s, "s")
    assert_equal(down(xs), xs_ref, "x_scale")
    assert_equal(down(xq), xq_ref, "x_q")
    assert_equal(down(sw), sw_ref, "w_scale")
    assert_equal(down(wq), wq_ref, "w_q")


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_act_extreme_ranges(orc, dtype, tiled):
    xt, s = _extreme_case(dtype)
    m, k = xt.f32.shape
    with np.errstate(over="raise", invalid="raise"):
        q = xt.f32.astype(np.float64) / s.astype(np.float64)[None, :]
    assert np.isfinite(q).all() and np.abs(q).max() < 2.0 ** 127
    assert (np.abs(q[q != 0]) < 2.0 ** -50).any() and (np.abs(q) > 2.0 ** 120).any()
    xs = _zeros(m, torch.float32)
    if tiled:
        xq = B.tiled_empty(m, k, DEV)
        B.sq_quantize_act_tiled(up(xt), up(s), xq, xs)
        xq = B.untile(xq, m, k)
    else:
        xq = _zeros((m, k), torch.int8)
        B.sq_quantize_act(up(xt), up(s), xq, xs)
    torch.cuda.synchronize()
    xq_ref, xs_ref = orc.quantize_act(xt.f32, s)
    assert_equal(down(xs), xs_ref, "x_scale")
    assert_equal(down(xq), xq_ref, "x_q")


# ---------------------------------------------------------------------------
# a8-a9: int8 GEMM, raw int32 and dequantised
# ---------------------------------------------------------------------------
def _codes(rng, r, k):
    q = rng.integers(-127, 128, size=(r, k)).astype(np.int8)
    if r > 1:
        q[0] = -128  # extremes: |acc| = 128^2 k
    return q


GEMM_SHAPES = SMALL + [(256, 256, 64), (384, 640, 1024), (1000, 1000, 336)]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=_id)
def test_gemm_int32(orc, shape):
    m, n, k = shape
    rng = np.random.default_rng(m * 7 + n * 13 + k)
    a, b = _codes(rng, m, k), _codes(rng, n, k)
    y = _zeros((m, n), torch.int32)
    B.sq_w8a8_gemm(up(a), None, up(b), None, None, y)
    torch.cuda.synchronize()
    assert_equal(down(y), orc.int_gemm(a, b), "acc")


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 5, 32), (130, 260, 528), (257, 300, 1040), (1000, 1000, 336)], ids=_id)
def test_gemm_dequant(orc, shape, out, bias):
    m, n, k = shape
    rng = np.random.default_rng(m + n + k)
    a, b = _codes(rng, m, k), _codes(rng, n, k)
    sx = (rng.random(m, dtype=np.float32) * np.float32(0.05)).astype(np.float32)
    sw = (rng.random(n, dtype=np.float32) * np.float32(0.001)).astype(np.float32)
    bias_t = bias_f = None
    if bias is not None:
        bf = rng.standard_normal(n, dtype=np.float32) * np.float32(3.0)
        if bias == "bf16":
            bits = inputs.bf16_bits(bf)
            bias_f, bias_t = inputs.bf16_to_f32(bits), up(bits)
        else:
            bias_f, bias_t = bf, up(bf)
    y = _zeros((m, n), torch.float32 if out == "f32" else torch.bfloat16)
    B.sq_w8a8_gemm(up(a), up(sx), up(b), up(sw), bias_t, y)
    torch.cuda.synchronize()
    acc = orc.int_gemm(a, b)
    yref = orc.dequant(acc, sx, sw, bias_f)
    scale = np.abs(acc.astype(np.float64) * sx[:, None] * sw[None, :])
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if out == "f32":
        assert_f32_rel(down(y), yref, scale)
    elif bias_f is None:
        # without a bias nothing cancels: the strict 1-ulp bar applies
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref))
    else:
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref), yref, scale)


# ---------------------------------------------------------------------------
# Degenerate weights: an all-zero output row (its scale is the floor over
# 127, 0x2EAD26C5, and its codes are zero: quantize_per_channel_symmetric's
# clamp(min=1e-8)) and an all-zero input column (its maximum is the floor),
# through every entry point that prepares weights
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("alpha", [0.5, 0.3, None], ids=lambda a: f"a{a}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(24, 40, 272), (70, 300, 1040)], ids=_id)
def test_zero_weight_rows_and_columns(orc, shape, dtype, alpha):
    m, n, k = shape
    c = _case(shape, dtype)
    wf = c.w.f32.copy()
    wf[3] = 0.0                      # all-zero output rows
    wf[n - 1] = 0.0
    wf[:, 5] = 0.0                   # all-zero input columns
    wf[:, k - 16:k - 13] = 0.0
    wt = inputs.Tensor(wf, None if c.w.bits is None else inputs.bf16_bits(wf))
    xf = c.x.f32.copy()
    xf[:, k - 16] = 0.0              # one of them never seen in calibration either
    mx = orc.calibrate(xf)
    a = 0.5 if alpha is None else alpha
    mxa = None if alpha is None else mx
    mw_ref = orc.weight_col_max(wf)
    s_ref = orc.smoothing_factor(mxa, mw_ref, a)
    zero_scale = np.array([0x2EAD26C5], np.uint32).view(np.float32)[0]

    def check(s_dev, wq_np, ws_dev, what):
        s_gpu = down(s_dev)
        if alpha == 0.3:
            ulps = np.abs(s_gpu.view(np.int32).astype(np.int64) - s_ref.view(np.int32))
            assert ulps.max() <= 1, what
        else:
            assert_equal(s_gpu, s_ref, f"s ({what})")
        wq_ref, ws_ref = orc.quantize_rows(orc.smooth_weight(wf, s_gpu))
        assert ws_ref[3] == zero_scale and ws_ref[n - 1] == zero_scale
        assert not wq_ref[3].any() and not wq_ref[n - 1].any()
        assert not wq_ref[:, 5].any() and not wq_ref[:, k - 16:k - 13].any()
        assert_equal(down(ws_dev), ws_ref, f"w_scale ({what})")
        assert_equal(wq_np, wq_ref, f"w_q ({what})")

    w_dev = up(wt)
    mx_dev = None if mxa is None else up(mx)
    # sq_prepare_weight and its tiled twin
    s1, wq1, ws1 = _zeros(k, torch.float32), _zeros((n, k), torch.int8), _zeros(n, torch.float32)
    B.sq_prepare_weight(w_dev, mx_dev, a, s1, wq1, ws1)
    s2, wq2, ws2 = _zeros(k, torch.float32), B.tiled_empty(n, k, DEV), _zeros(n, torch.float32)
    B.sq_prepare_weight_tiled(w_dev, mx_dev, a, s2, wq2, ws2)
    # the split calls: column max, smoothing factor, weight codes
    mw = _zeros(k, torch.float32)
    B.sq_weight_col_max(w_dev, mw)
    s3 = _zeros(k, torch.float32)
    B.sq_smoothing_factor(mx_dev, mw, a, s3)
    wq3, ws3 = _zeros((n, k), torch.int8), _zeros(n, torch.float32)
    B.sq_quantize_weight(w_dev, s3, wq3, ws3)
    # re-smoothing from the stored maxima
    s4, wq4, ws4 = _zeros(k, torch.float32), _zeros((n, k), torch.int8), _zeros(n, torch.float32)
    B.sq_recompute_smooth_scale(w_dev, mx_dev, mw, a, s4, wq4, ws4)
    torch.cuda.synchronize()
    assert_equal(down(mw), mw_ref, "weight column max")
    assert mw_ref[5] == np.float32(1e-8)
    check(s1, down(wq1), ws1, "prepare")
    check(s2, down(B.untile(wq2, n, k)), ws2, "prepare tiled")
    check(s3, down(wq3), ws3, "split calls")
    check(s4, down(wq4), ws4, "recompute")


# ---------------------------------------------------------------------------
# a6-a9 in one call, with the workspace codes checked too
# ---------------------------------------------------------------------------
def _check_linear(orc, c, s, wq, sw, x_dev, bias_dev, out_dtype, rows=None):
    m, n, k = c.m, c.n, c.k
    y = _zeros((m, n), out_dtype)
    ws = torch.empty(B.sq_w8a8_linear_workspace_bytes(m, k), dtype=torch.uint8, device=DEV)
    B.sq_w8a8_linear(x_dev, up(s), up(wq), up(sw), bias_dev, y, ws)
    torch.cuda.synchronize()
    xq_gpu, xs_gpu = (down(t) for t in B.workspace_views(ws, m, k))
    xq_ref, xs_ref = orc.quantize_act(c.x.f32, s)
    assert_equal(xs_gpu, xs_ref, "x_scale (linear)")
    assert_equal(xq_gpu, xq_ref, "x_q (linear)")
    sel = np.arange(m) if rows is None else rows
    acc = orc.int_gemm(xq_ref[sel], wq)
    bias_f = None if c.bias is None else c.bias.f32
    yref = orc.dequant(acc, xs_ref[sel], sw, bias_f)
    ysel = down(y[torch.from_numpy(sel).to(DEV)])
    scale = np.abs(acc.astype(np.float64) * xs_ref[sel][:, None] * sw[None, :])
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if out_dtype == torch.float32:
        assert_f32_rel(ysel, yref, scale)
    else:
        # without a bias nothing cancels: the strict 1-ulp bar applies
        if bias_f is None:
            assert_bf16_within_one_ulp(ysel, orc.to_bf16(yref))
        else:
            assert_bf16_within_one_ulp(ysel, orc.to_bf16(yref), yref, scale)
    return y


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_linear(orc, shape, dtype):
    c = _case(shape, dtype)
    s, wq, sw = orc.prepare_weight(c.w.f32, orc.calibrate(c.x.f32), 0.5)
    out = torch.float32 if dtype == "f32" else torch.bfloat16
    y1 = _check_linear(orc, c, s, wq, sw, up(c.x), upo(c.bias), out)
    y2 = _check_linear(orc, c, s, wq, sw, up(c.x), upo(c.bias), out)
    assert torch.equal(y1.view(torch.int16 if out == torch.bfloat16 else torch.int32),
                       y2.view(torch.int16 if out == torch.bfloat16 else torch.int32)), "not deterministic"


def test_golden_hand_example_on_gpu():
    """The hand-derived example (ties included), padded to k = 16 with zero
    channels (floored: s = 1 there, codes 0), through the whole GPU path."""
    d = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_alpha_half.json")))
    ex = d["expected"]
    for dtype in ("f32", "bf16"):
        x = np.zeros((3, 16), np.float32)
        x[:, :4] = d["x"]
        w = np.zeros((2, 16), np.float32)
        w[:, :4] = d["w"]
        b = np.array(d["bias"], np.float32)
        xt = inputs.Tensor(x, inputs.bf16_bits(x) if dtype == "bf16" else None)
        wt = inputs.Tensor(w, inputs.bf16_bits(w) if dtype == "bf16" else None)
        bt = inputs.Tensor(b, inputs.bf16_bits(b) if dtype == "bf16" else None)
        run = _zeros(16, torch.float32)
        B.sq_calibrate(up(xt), run)
        smooth, wq, ws = _zeros(16, torch.float32), _zeros((2, 16), torch.int8), _zeros(2, torch.float32)
        B.sq_prepare_weight(up(wt), run, d["alpha"], smooth, wq, ws)
        y = _zeros((3, 2), torch.float32)
        wsp = torch.empty(B.sq_w8a8_linear_workspace_bytes(3, 16), dtype=torch.uint8, device=DEV)
        B.sq_w8a8_linear(up(xt), smooth, wq, ws, up(bt), y, wsp)
        torch.cuda.synchronize()
        assert np.array_equal(down(run)[:4], np.array(ex["mx"], np.float32))
        assert np.array_equal(down(smooth), np.array(ex["s"] + [1.0] * 12, np.float32))
        assert np.array_equal(down(wq)[:, :4], np.array(ex["wq"])) and not down(wq)[:, 4:].any()
        xq, xs = (down(t) for t in B.workspace_views(wsp, 3, 16))
        assert np.array_equal(xq[:, :4], np.array(ex["xq"])) and not xq[:, 4:].any()
        assert np.array_equal(xs, np.array(ex["scale_x"], np.float32))
        assert np.array_equal(down(y), np.array(ex["y"], np.float32))
        yi = _zeros((3, 2), torch.int32)
        B.sq_w8a8_gemm(up(xq), None, wq, None, None, yi)
        torch.cuda.synchronize()
        assert np.array_equal(down(yi), np.array(ex["acc"]))


def test_layer_lifecycle():
    """The page's state machine on top of the ABI: calibrate -> freeze ->
    forward; calibrating after the freeze raises."""
    c = _case((40, 24, 64), "bf16")
    layer = B.SmoothQuantLinear(up(c.w), upo(c.bias), alpha=0.5)
    layer.calibrate(up(c.x)[:20])
    layer.calibrate(up(c.x)[20:])
    assert layer.freeze() == B.SQ_OK
    with pytest.raises(RuntimeError):
        layer.calibrate(up(c.x))
    y = layer.forward(up(c.x))
    assert y.shape == (40, 24) and y.dtype == torch.bfloat16
    fresh = B.SmoothQuantLinear(up(c.w), None)
    assert fresh.freeze() == B.SQ_WARN_UNCALIBRATED
    assert torch.all(fresh.smooth == 1.0)


@pytest.mark.parametrize("rows", [[128, 128, 128, 128], [3, 0, 90]], ids=["4x128", "ragged"])
def test_calibrate_batches_graph_replays(orc, rows):
    """sq_calibrate_batches captured in a HIP graph (its zero fill is a
    kernel, not a memset) and replayed four times, the buffer refilled with
    values above every |x| and other work run eagerly between replays:
    every replay gives the oracle's running max."""
    k = 4096
    total = sum(rows)
    c = inputs.small(total, 8, k, seed=total + 5, dtype="bf16", bias=False)
    x = up(c.x)
    cuts = np.cumsum([0] + rows)
    batches = [x[a:b].clone() for a, b in zip(cuts[:-1], cuts[1:])]
    want = orc.calibrate(c.x.f32)
    run = torch.full((k,), 1e30, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(DEV)
    stream.wait_stream(torch.cuda.current_stream())
    call = B.prepared(B.sq_calibrate_batches, batches, run, True, stream)
    with torch.cuda.stream(stream):
        call()  # eager once before capture
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    other = torch.zeros(k, dtype=torch.float32, device=DEV)
    for i in range(4):
        run.fill_(1e30 + i)
        other += 1.0  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_equal(down(run), want, f"running max, replay {i}")


def test_layer_calibrate_batches(orc):
    """SmoothQuantLinear.calibrate_batches: eleven batches (two calls of
    sq_calibrate_batches, the first starting the running max, one batch
    empty) give the oracle's running max over all their rows, and then the
    same smoothing factor and codes as the layer calibrated batch by batch."""
    c = _case((300, 24, 272), "bf16")
    x = up(c.x)
    cuts = [0, 1, 30, 30, 64, 100, 128, 160, 200, 233, 260, 300]
    batches = [x[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    many = B.SmoothQuantLinear(up(c.w), None, alpha=0.5)
    many.calibrate(x[:0])  # an empty first batch starts nothing
    many.calibrate_batches(batches)
    one = B.SmoothQuantLinear(up(c.w), None, alpha=0.5)
    for b in batches:
        one.calibrate(b)
    torch.cuda.synchronize()
    assert many.calib_count == one.calib_count == 300
    assert_equal(down(many.calib_max_abs), orc.calibrate(c.x.f32), "running max")
    many.freeze()
    one.freeze()
    torch.cuda.synchronize()
    assert torch.equal(many.smooth, one.smooth) and torch.equal(many.weight_int8, one.weight_int8)


@pytest.mark.parametrize("layout", ["row", "tiled"])
def test_layer_fp32_weights_bf16_activations(orc, layout):
    """fp32 weights and bias with bf16 activations: the forward takes the
    bias in its own type on both layouts (the same bits), and
    quantization_error widens the bf16 activations (exactly) rather than
    narrowing the weights."""
    c32 = inputs.small(40, 24, 272, seed=91, dtype="f32", bias=True)
    cb = inputs.small(40, 24, 272, seed=91, dtype="bf16", bias=False)
    x_bits = cb.x.bits
    x_f = cb.x.f32                                  # bf16 values, exactly
    layer = B.SmoothQuantLinear(up(c32.w), up(c32.bias), alpha=0.5, layout=layout)
    layer.calibrate(up(x_bits))
    assert layer.freeze() == B.SQ_OK
    y = layer.forward(up(x_bits), out_dtype=torch.float32)
    torch.cuda.synchronize()
    mx = orc.calibrate(x_f)
    s, wq, sw = orc.prepare_weight(c32.w.f32, mx, 0.5)
    xq, sx, acc, yref = orc.linear(x_f, s, wq, sw, c32.bias.f32)
    scale = np.abs(acc.astype(np.float64) * sx[:, None] * sw[None, :]) + np.abs(c32.bias.f32)[None, :]
    assert_f32_rel(down(y), yref, scale)
    # the bound the two outputs' own tolerances give (as for the layer's
    # quantization_error below): y_q within 1e-6 (|acc sx sw| + |bias|),
    # y_fp (fp32 operands) within (k + 1) 2^-24 sum|x w| + 2^-24 |y_fp|
    got = layer.quantization_error(up(x_bits))
    yfp = orc.reference_linear(x_f, c32.w.f32, c32.bias.f32)
    want = orc.relative_error(yfp, yref)[0]
    bfp = (c32.k + 1) * 2.0 ** -24 * (np.abs(x_f.astype(np.float64)) @ np.abs(c32.w.f32.astype(np.float64)).T)
    bfp = bfp + 2.0 ** -24 * np.abs(yfp)
    tol = (np.linalg.norm(1e-6 * scale) + np.linalg.norm(bfp)) / np.linalg.norm(yfp)
    assert abs(got - want) <= tol + 1e-12, (got, want, tol)


def test_hardware_reciprocal_is_correctly_rounded():
    """The activation path's 1/s (hardware reciprocal + one Newton step)
    equals the IEEE quotient for every binary32 s in [2^-100, 2^100)."""
    cnt = _zeros(1, torch.int64)
    B.sq_selfcheck_reciprocal(cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0


def test_division_scheme_is_correctly_rounded():
    """The quantisation kernels' quotient (RN(1/b), then one fma correction)
    equals the IEEE quotient for all 2^46 pairs of binary32 significands,
    swept in 8 launches of 2^20 divisors each."""
    cnt = _zeros(1, torch.int64)
    step = 1 << 20
    for b0 in range(0, 1 << 23, step):
        B.sq_selfcheck_division(b0, b0 + step, cnt)
        torch.cuda.synchronize()
        print(f"divisor significands [{b0}, {b0 + step}): {int(cnt.item())} mismatches so far", flush=True)
    assert int(cnt.item()) == 0


# ---------------------------------------------------------------------------
# a8-a9 for few tokens (m <= 64: the weight-streaming kernel): token counts
# around every 16-row group, weight rows around every 16-row block, K tails
# of 16/32/48 bytes and K long enough for several rounds of every wavefront,
# weight rows over several workgroups of up to 48; m = 65 and 80 cross over
# to the tiled kernel.
# ---------------------------------------------------------------------------
STREAM = [(1, 1, 16), (2, 17, 48), (15, 16, 64), (16, 100, 208), (17, 31, 4096), (31, 15, 1040),
          (32, 33, 11008), (33, 64, 80), (48, 47, 336), (49, 200, 2048), (63, 65, 4112),
          (64, 129, 4096), (16, 12289, 272), (64, 4099, 1040), (65, 70, 272), (80, 33, 4096)]


@pytest.mark.parametrize("shape", STREAM, ids=_id)
def test_stream_int32(orc, shape):
    m, n, k = shape
    rng = np.random.default_rng(m * 31 + n * 17 + k)
    a, b = _codes(rng, m, k), _codes(rng, n, k)
    y = _zeros((m, n), torch.int32)
    B.sq_w8a8_gemm(up(a), None, up(b), None, None, y)
    torch.cuda.synchronize()
    assert_equal(down(y), orc.int_gemm(a, b), "acc")


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 33, 64), (16, 200, 4096), (37, 129, 1040), (64, 100, 528)], ids=_id)
def test_stream_dequant(orc, shape, out, bias):
    test_gemm_dequant(orc, shape, out, bias)


# ---------------------------------------------------------------------------
# Per-tensor variant (page "quantized_linear.py": quantize_tensor,
# QuantizedLinear): one scale per tensor, replaced by 1 below 1e-8
# ---------------------------------------------------------------------------
TENSOR_SHAPES = [(1, 16), (3, 48), (130, 528), (257, 1040), (1000, 4096)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", TENSOR_SHAPES, ids=_id)
def test_quantize_tensor(orc, shape, dtype):
    m, k = shape
    c = inputs.small(m, 8, k, seed=11 + m + k, dtype=dtype, bias=False)
    q = _zeros((m, k), torch.int8)
    sc = _zeros(1, torch.float32)
    B.sq_quantize_tensor(up(c.x), q, sc)
    torch.cuda.synchronize()
    q_ref, sc_ref = orc.quantize_tensor(c.x.f32)
    assert_equal(down(sc)[0], sc_ref, "scale")
    assert_equal(down(q), q_ref, "codes")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_tensor_replacement(orc, dtype):
    """An all-zero tensor and one whose max / 127 is below 1e-8 both get the
    scale 1 (and zero codes); just above, the scale is max / 127."""
    for v in (np.zeros((4, 32), np.float32),
              np.full((2, 16), 1e-6, np.float32) * np.linspace(-1, 1, 32, dtype=np.float32).reshape(2, 16),
              np.full((2, 16), 2e-6, np.float32) * np.linspace(-1, 1, 32, dtype=np.float32).reshape(2, 16)):
        if dtype == "bf16":
            bits = inputs.bf16_bits(v)
            v, x_dev = inputs.bf16_to_f32(bits), up(bits)
        else:
            x_dev = up(v)
        q = _zeros(v.shape, torch.int8)
        sc = _zeros(1, torch.float32)
        B.sq_quantize_tensor(x_dev, q, sc)
        torch.cuda.synchronize()
        q_ref, sc_ref = orc.quantize_tensor(v)
        assert_equal(down(sc)[0], sc_ref, "scale")
        assert_equal(down(q), q_ref, "codes")


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 5, 32), (16, 200, 4096), (64, 129, 528), (130, 260, 528),
                                   (257, 300, 1040)], ids=_id)
def test_gemm_per_tensor(orc, shape, out, bias):
    """Codes and scales from sq_quantize_tensor, then the per-tensor product
    (both kernels: m <= 64 streams the weights, larger m is tiled)."""
    m, n, k = shape
    c = inputs.small(m, n, k, seed=5 + m + n + k, dtype="bf16", bias=bias is not None)
    x_dev, w_dev = up(c.x), up(c.w)
    xq, sx = _zeros((m, k), torch.int8), _zeros(1, torch.float32)
    wq, sw = _zeros((n, k), torch.int8), _zeros(1, torch.float32)
    B.sq_quantize_tensor(x_dev, xq, sx)
    B.sq_quantize_tensor(w_dev, wq, sw)
    bias_f = bias_t = None
    if bias == "f32":
        bias_f = c.bias.f32
        bias_t = up(bias_f)
    elif bias == "bf16":
        bias_f, bias_t = c.bias.f32, up(c.bias)
    y = _zeros((m, n), torch.float32 if out == "f32" else torch.bfloat16)
    B.sq_w8a8_gemm_per_tensor(xq, sx, wq, sw, bias_t, y)
    torch.cuda.synchronize()
    xq_ref, sx_ref, wq_ref, sw_ref, acc, yref = orc.linear_per_tensor(c.x.f32, c.w.f32, bias_f)
    assert_equal(down(xq), xq_ref, "x codes")
    assert_equal(down(wq), wq_ref, "w codes")
    scale = np.abs(acc.astype(np.float64) * float(sx_ref) * float(sw_ref))
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if out == "f32":
        assert_f32_rel(down(y), yref, scale)
    else:
        # the cancellation allowance only with a bias; without one the strict 1-ulp bar
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref), *(() if bias_f is None else (yref, scale)))


# ---------------------------------------------------------------------------
# Weight-only int8 linear (torchao page "quantization/subclass.py",
# Int8WeightOnlyQuantizedLinearWeight): bf16 activations x int8 weights.
# Tolerance from the arithmetic: the products are exact in fp32 and the sum
# of K of them, in any order, is within K * 2^-24 * sum |x w| of the exact
# sum; the scale multiply and the bias add round once each (2^-24 of their
# result each), and a bf16 output adds half a bf16 ulp.
# ---------------------------------------------------------------------------
def _assert_wo_close(got_bits_or_f32, yref, mag, k, out):
    if out == "f32":
        got = got_bits_or_f32.astype(np.float64)
        half_ulp = 0.0
    else:
        got = (got_bits_or_f32.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        e = np.floor(np.log2(np.maximum(np.abs(yref), 2.0 ** -126)))
        half_ulp = 2.0 ** (e - 8)
    bound = k * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(yref) + half_ulp + 1e-30
    err = np.abs(got - yref)
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), float((err / bound).max()))


WO_SHAPES = [(1, 1, 16), (3, 17, 48), (16, 100, 272), (16, 200, 4096), (33, 64, 528), (64, 129, 1040),
             (80, 70, 256), (130, 40, 4112)]


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", WO_SHAPES, ids=_id)
def test_wo_linear(orc, shape, out, bias):
    m, n, k = shape
    rng = np.random.default_rng(m * 3 + n * 5 + k)
    c = inputs.small(m, n, k, seed=21 + m + n + k, dtype="bf16", bias=bias is not None)
    wq = _codes(rng, n, k)
    sw = (rng.random(n, dtype=np.float32) * np.float32(0.002) + np.float32(1e-4)).astype(np.float32)
    bias_f = bias_t = None
    if bias == "f32":
        bias_f = c.bias.f32
        bias_t = up(bias_f)
    elif bias == "bf16":
        bias_f, bias_t = c.bias.f32, up(c.bias)
    y = _zeros((m, n), torch.float32 if out == "f32" else torch.bfloat16)
    B.sq_wo_linear(up(c.x), up(wq), up(sw), bias_t, y)
    torch.cuda.synchronize()
    yref = orc.wo_linear(c.x.f32, wq, sw, bias_f)
    mag = (np.abs(c.x.f32.astype(np.float64)) @ np.abs(wq.astype(np.float64)).T) * sw[None, :].astype(np.float64)
    _assert_wo_close(down(y), yref, mag, k, out)


# ---------------------------------------------------------------------------
# Re-smoothing from stored maxima and quantization_error (page
# "w8a8_smoothquant.py": recompute_smooth_scale, quantization_error).
# ---------------------------------------------------------------------------
def _with_zero_column(t, dtype):
    """The weights of a case with input channel 0 all zero (floored max)."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(t.bits).copy()
        bits[:, 0] = 0
        f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return up(bits), f32
    f32 = t.f32.copy()
    f32[:, 0] = 0.0
    return up(f32), f32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_weight_col_max(orc, shape, dtype):
    c = _case(shape, dtype)
    w, w_np = _with_zero_column(c.w, dtype)
    mw = torch.full((c.k,), -1.0, dtype=torch.float32, device=DEV)
    assert B.sq_weight_col_max(w, mw) == B.SQ_OK
    torch.cuda.synchronize()
    want = orc.weight_col_max(w_np)
    assert want[0] == np.float32(1e-8)
    assert_equal(down(mw), want, "weight column max")


@pytest.mark.parametrize("alpha", ALPHAS, ids=lambda a: f"a{a}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(7, 17, 48), (130, 260, 528), (64, 512, 4096), (5, 40, 11008)], ids=_id)
def test_recompute_smooth_scale(orc, shape, dtype, alpha):
    c = _case(shape, dtype)
    w = up(c.w)
    mx = orc.calibrate(c.x.f32)
    mw = _zeros(c.k, torch.float32)
    B.sq_weight_col_max(w, mw)
    s, wq, sw = _zeros(c.k, torch.float32), _zeros((c.n, c.k), torch.int8), _zeros(c.n, torch.float32)
    # a stale result of another alpha first: every output must be rewritten
    B.sq_recompute_smooth_scale(w, up(mx), mw, 0.9, s, wq, sw)
    st = B.sq_recompute_smooth_scale(w, None if alpha is None else up(mx), mw, 0.5 if alpha is None else alpha,
                                     s, wq, sw)
    torch.cuda.synchronize()
    assert st == (B.SQ_WARN_UNCALIBRATED if alpha is None else B.SQ_OK)
    s_ref, wq_ref, sw_ref = orc.prepare_weight(c.w.f32, None if alpha is None else mx,
                                               0.5 if alpha is None else alpha)
    assert_equal(down(s), s_ref, "smooth")
    assert_equal(down(sw), sw_ref, "w_scale")
    assert_equal(down(wq), wq_ref, "w_q")


def _assert_sum_close(got, yref, mag, terms, out):
    """An fp32 sum of `terms` rounded terms (any order) is within
    terms 2^-24 sum|term| of the exact sum; the bias add rounds once more,
    a bf16 output adds half a bf16 ulp."""
    if out == "f32":
        g = got.astype(np.float64)
        half_ulp = 0.0
    else:
        g = (got.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        e = np.floor(np.log2(np.maximum(np.abs(yref), 2.0 ** -126)))
        half_ulp = 2.0 ** (e - 8)
    bound = terms * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(yref) + half_ulp + 1e-30
    err = np.abs(g - yref)
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), float((err / bound).max()))


REF = [(1, 1, 16), (3, 17, 48), (33, 7, 272), (130, 260, 528), (257, 300, 1040), (300, 129, 2064)]


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", REF, ids=_id)
def test_reference_linear(orc, shape, dtype, out, bias):
    m, n, k = shape
    c = _case(shape, dtype, seed=31, bias=True)
    bias_t = bias_f = None
    if bias == "f32":
        bias_f = c.bias.f32.astype(np.float32)
        bias_t = up(bias_f)
    elif bias == "bf16":
        bt = torch.from_numpy(c.bias.f32.astype(np.float32)).to(torch.bfloat16)
        bias_f = bt.float().numpy()
        bias_t = bt.to(DEV)
    y = _zeros((m, n), torch.float32 if out == "f32" else torch.bfloat16)
    assert B.sq_reference_linear(up(c.x), up(c.w), bias_t, y) == B.SQ_OK
    torch.cuda.synchronize()
    yref = orc.reference_linear(c.x.f32, c.w.f32, bias_f)
    mag = np.abs(c.x.f32.astype(np.float64)) @ np.abs(c.w.f32.astype(np.float64)).T
    _assert_sum_close(down(y), yref, mag, k + 1 if dtype == "f32" else k, out)


@pytest.mark.parametrize("count", [1, 3, 4, 1000, 4099, (1 << 20) + 5, 3 * (1 << 22) + 1])
def test_relative_error(orc, count):
    rng = np.random.default_rng(count)
    a = rng.standard_normal(count, dtype=np.float32)
    b = (a + rng.standard_normal(count, dtype=np.float32) * np.float32(0.01)).astype(np.float32)
    ws = torch.empty(max(B.sq_relative_error_workspace_bytes(count), 8), dtype=torch.uint8, device=DEV)
    res = torch.empty(3, dtype=torch.float64, device=DEV)
    a_d, b_d = up(a), up(b)
    assert B.sq_relative_error(a_d, b_d, ws, res) == B.SQ_OK
    got = down(res).copy()
    ratio, num, den = orc.relative_error(a.astype(np.float64), b.astype(np.float64))
    # a sum of `count` non-negative binary64 terms is within (count - 1) 2^-53
    # of the exact sum relative to it, in any order (the oracle's sequential
    # sum and the kernel's blocked one each); a square root halves a relative
    # error, the ratio adds two
    tol = (count + 64) * 2.0 ** -53
    for g, w, t in zip(got, (num, den, ratio), (tol, tol, 2 * tol)):
        assert abs(g - w) <= t * abs(w), (g, w)
    # the same count gives the same bits
    B.sq_relative_error(a_d, b_d, ws, res)
    assert np.array_equal(down(res).view(np.uint64), got.view(np.uint64))
    # a zero reference: the denominator floor
    zero = _zeros(count, torch.float32)
    B.sq_relative_error(zero, b_d, ws, res)
    got = down(res)
    ratio, num, den = orc.relative_error(np.zeros(count), b.astype(np.float64))
    assert got[1] == 0.0 and den == 0.0
    assert abs(got[0] - num) <= tol * num and abs(got[2] - ratio) <= 2 * tol * ratio


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_quantization_error(orc, dtype):
    """The layer's quantization_error (reference linear, quantized forward in
    fp32, relative error) against the oracle's, within the bound the two
    outputs' own tolerances give: y_q within 1e-6 (|acc sx sw| + |bias|),
    y_fp within (k + 1) 2^-24 sum|x w| + 2^-24 |y_fp|."""
    c = inputs.tiny() if dtype == "f32" else inputs.small(48, 96, 272, seed=5, dtype="bf16")
    layer = B.SmoothQuantLinear(up(c.w), up(c.bias), alpha=0.5)
    layer.calibrate(up(c.x))
    layer.freeze()
    mx = orc.calibrate(c.x.f32)
    x64, w64 = c.x.f32.astype(np.float64), c.w.f32.astype(np.float64)
    for alpha in (0.5, 0.25, 1.0, 0.0):
        layer.recompute(alpha)
        got = layer.quantization_error(up(c.x))
        want = orc.quantization_error(c.x.f32, c.w.f32, c.bias.f32, mx, alpha)
        s, wq, sw = orc.prepare_weight(c.w.f32, mx, alpha)
        xq, sx, acc, y = orc.linear(c.x.f32, s, wq, sw, c.bias.f32)
        yfp = orc.reference_linear(c.x.f32, c.w.f32, c.bias.f32)
        bq = 1e-6 * (np.abs(acc * sx[:, None].astype(np.float64) * sw[None, :]) + np.abs(c.bias.f32)[None, :])
        bfp = (c.k + 1) * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T) + 2.0 ** -24 * np.abs(yfp)
        tol = (np.linalg.norm(bq) + np.linalg.norm(bfp)) / np.linalg.norm(yfp)
        assert abs(got - want) <= tol + 1e-12, (alpha, got, want, tol)


@pytest.mark.parametrize("alpha", ALPHAS, ids=lambda a: f"a{a}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(7, 17, 48), (130, 260, 528), (64, 512, 4096), (5, 40, 11008)], ids=_id)
def test_split_prepare(orc, shape, dtype, alpha):
    """sq_weight_col_max -> sq_smoothing_factor -> sq_quantize_weight (the
    weight preparation as separate calls, the column max on a second stream)
    equals the oracle's preparation bit for bit."""
    c = _case(shape, dtype)
    w = up(c.w)
    mx = orc.calibrate(c.x.f32)
    side = torch.cuda.Stream()
    mw = _zeros(c.k, torch.float32)
    # the side stream starts after the inputs and the zero fill are done
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.sq_weight_col_max(w, mw)
    torch.cuda.current_stream().wait_stream(side)
    s, wq, sw = _zeros(c.k, torch.float32), _zeros((c.n, c.k), torch.int8), _zeros(c.n, torch.float32)
    st = B.sq_smoothing_factor(None if alpha is None else up(mx), mw, 0.5 if alpha is None else alpha, s)
    assert st == (B.SQ_WARN_UNCALIBRATED if alpha is None else B.SQ_OK)
    assert B.sq_quantize_weight(w, s, wq, sw) == B.SQ_OK
    torch.cuda.synchronize()
    s_ref, wq_ref, sw_ref = orc.prepare_weight(c.w.f32, None if alpha is None else mx,
                                               0.5 if alpha is None else alpha)
    assert_equal(down(s), s_ref, "smooth")
    assert_equal(down(sw), sw_ref, "w_scale")
    assert_equal(down(wq), wq_ref, "w_q")
