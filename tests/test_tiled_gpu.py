"""GPU parity of the tiled int8 layout (16 x 64 tiles): the activation and
weight codes written in tiles (sq_quantize_act_tiled, sq_prepare_weight_tiled)
and the int8 product read from them (sq_w8a8_gemm_tiled), against the CPU
oracle on seeded inputs.

The codes, once untiled, are compared with the oracle bit for bit, and the
padding columns of every stored row must hold zero codes (the product sums
over them). The product's int32 results are compared bit for bit; fp32 and
bf16 outputs to the same bar as the row-major product (fp32 within 1e-6 of
|acc sx sw| + |bias|, bf16 within one ulp of the oracle's binary64 result
rounded once). The tiled operands of the product are built on the host here,
with random bytes in the padding rows, which no stored output may read."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_bf16_within_one_ulp, assert_equal, assert_f32_rel, down, require_gpu, up
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import inputs

pytestmark = pytest.mark.gpu

# single elements, ragged row groups and K tails (k % 64 of 16, 32, 48),
# several 256-row tiles, the largest K
SMALL = [(1, 1, 16), (3, 5, 32), (7, 17, 48), (17, 33, 272), (33, 7, 16), (130, 260, 528),
         (257, 300, 1040), (64, 512, 4096), (5, 40, 11008), (300, 129, 2064), (70, 33, 16384)]
GEMM_SHAPES = SMALL + [(256, 256, 64), (384, 640, 1024), (1000, 1000, 336), (513, 769, 4160), (48, 777, 208),
                       (16, 11008, 4096)]


def _id(s):
    return "x".join(map(str, s))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    B.lib()


def _tile_host(a: np.ndarray, rng) -> np.ndarray:
    """[rows][k] int8 codes into the flat 16 x 64 tiled layout: zero padding
    columns, random bytes in the padding rows."""
    rows, k = a.shape
    r16, k64 = (rows + 15) // 16 * 16, (k + 63) // 64 * 64
    p = rng.integers(-128, 128, size=(r16, k64)).astype(np.int8)
    p[:rows] = 0
    p[:rows, :k] = a
    return np.ascontiguousarray(p.reshape(r16 // 16, 16, k64 // 64, 64).transpose(0, 2, 1, 3)).reshape(-1)


def _garbage(rows, k):
    """A tiled buffer pre-filled with a non-zero byte, so that padding the
    kernel fails to clear shows up."""
    t = B.tiled_empty(rows, k, DEV)
    t.fill_(0x5A)
    return t


def _padding_columns(t: torch.Tensor, rows: int, k: int) -> np.ndarray:
    k64 = (k + 63) // 64 * 64
    full = down(B.untile(t, rows, k64))
    return full[:, k:]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL, ids=_id)
def test_quantize_act_tiled(orc, shape, dtype):
    m, n, k = shape
    c = inputs.small(m, n, k, seed=7 + m + 3 * n + k, dtype=dtype)
    s, _, _ = orc.prepare_weight(c.w.f32, orc.calibrate(c.x.f32), 0.5)
    xq = _garbage(m, k)
    xs = torch.zeros(m, dtype=torch.float32, device=DEV)
    B.sq_quantize_act_tiled(up(c.x), up(s), xq, xs)
    torch.cuda.synchronize()
    xq_ref, xs_ref = orc.quantize_act(c.x.f32, s)
    assert_equal(down(xs), xs_ref, "x_scale")
    assert_equal(down(B.untile(xq, m, k)), xq_ref, "x_q (untiled)")
    assert not _padding_columns(xq, m, k).any(), "padding columns not zero"


@pytest.mark.parametrize("alpha", [0.5, 0.3, None], ids=lambda a: f"a{a}")
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SMALL[::2] + [(64, 512, 4096), (300, 129, 2064)], ids=_id)
def test_prepare_weight_tiled(orc, shape, dtype, alpha):
    """Bit-identical to the row-major preparation (s, w_scale and the codes),
    and the codes to the oracle's."""
    m, n, k = shape
    c = inputs.small(m, n, k, seed=7 + m + 3 * n + k, dtype=dtype)
    w = up(c.w)
    mx = None if alpha is None else up(orc.calibrate(c.x.f32))
    a = 0.5 if alpha is None else alpha
    s_t = torch.zeros(k, dtype=torch.float32, device=DEV)
    sw_t = torch.zeros(n, dtype=torch.float32, device=DEV)
    wq_t = _garbage(n, k)
    st_t = B.sq_prepare_weight_tiled(w, mx, a, s_t, wq_t, sw_t)
    s_r = torch.zeros(k, dtype=torch.float32, device=DEV)
    sw_r = torch.zeros(n, dtype=torch.float32, device=DEV)
    wq_r = torch.zeros((n, k), dtype=torch.int8, device=DEV)
    st_r = B.sq_prepare_weight(w, mx, a, s_r, wq_r, sw_r)
    torch.cuda.synchronize()
    assert st_t == st_r == (B.SQ_WARN_UNCALIBRATED if alpha is None else B.SQ_OK)
    assert_equal(down(s_t), down(s_r), "s (tiled vs row-major)")
    assert_equal(down(sw_t), down(sw_r), "w_scale (tiled vs row-major)")
    assert_equal(down(B.untile(wq_t, n, k)), down(wq_r), "w_q (tiled vs row-major)")
    assert not _padding_columns(wq_t, n, k).any(), "padding columns not zero"
    s_gpu = down(s_t)
    wq_ref, ws_ref = orc.quantize_rows(orc.smooth_weight(c.w.f32.copy(), s_gpu))
    assert_equal(down(sw_t), ws_ref, "w_scale")
    assert_equal(down(B.untile(wq_t, n, k)), wq_ref, "w_q")


def _codes(rng, r, k):
    q = rng.integers(-127, 128, size=(r, k)).astype(np.int8)
    if r > 1:
        q[0] = -128  # extremes: |acc| = 128^2 k
    return q


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=_id)
def test_gemm_tiled_int32(orc, shape):
    m, n, k = shape
    print(f"tiled gemm int32 {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(m * 7 + n * 13 + k + 1)
    a, b = _codes(rng, m, k), _codes(rng, n, k)
    y = torch.zeros((m, n), dtype=torch.int32, device=DEV)
    B.sq_w8a8_gemm_tiled(up(_tile_host(a, rng)), None, m, up(_tile_host(b, rng)), None, n, k, None, y)
    torch.cuda.synchronize()
    assert_equal(down(y), orc.int_gemm(a, b), "acc")


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 5, 32), (16, 4099, 80), (64, 300, 1040), (130, 260, 528), (257, 300, 1040),
                                   (1000, 1000, 336)], ids=_id)
def test_gemm_tiled_dequant(orc, shape, out, bias):
    """Against the oracle, and bit for bit against the row-major product on
    the same codes: both compute the exact int32 sums and the same epilogue
    expression (f32(acc) * sx * sw, then + bias), whether the product runs
    on MFMA tiles (more than 64 rows) or streams the weights (64 or fewer)."""
    m, n, k = shape
    rng = np.random.default_rng(m + n + k + 1)
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
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y = torch.zeros((m, n), dtype=odt, device=DEV)
    B.sq_w8a8_gemm_tiled(up(_tile_host(a, rng)), up(sx), m, up(_tile_host(b, rng)), up(sw), n, k, bias_t, y)
    y_rm = torch.zeros((m, n), dtype=odt, device=DEV)
    B.sq_w8a8_gemm(up(a), up(sx), up(b), up(sw), bias_t, y_rm)
    torch.cuda.synchronize()
    acc = orc.int_gemm(a, b)
    yref = orc.dequant(acc, sx, sw, bias_f)
    scale = np.abs(acc.astype(np.float64) * sx[:, None] * sw[None, :])
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if out == "f32":
        assert_f32_rel(down(y), yref, scale)
    else:
        # the cancellation allowance only with a bias; without one the strict 1-ulp bar
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref), *(() if bias_f is None else (yref, scale)))
    assert_equal(down(y), down(y_rm), "tiled vs row-major")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 5, 32), (17, 33, 272), (130, 260, 528), (257, 300, 1040),
                                   (70, 33, 16384), (16, 11008, 4096), (64, 1000, 4160), (1, 4096, 11008)],
                         ids=_id)
def test_linear_tiled(orc, shape, dtype):
    """The three tiled calls in a row, as a layer runs them."""
    m, n, k = shape
    c = inputs.small(m, n, k, seed=11 + m + n + k, dtype=dtype)
    mx = orc.calibrate(c.x.f32)
    s = torch.empty(k, dtype=torch.float32, device=DEV)
    wq = B.tiled_empty(n, k, DEV)
    sw = torch.empty(n, dtype=torch.float32, device=DEV)
    B.sq_prepare_weight_tiled(up(c.w), up(mx), 0.5, s, wq, sw)
    xq = B.tiled_empty(m, k, DEV)
    xs = torch.empty(m, dtype=torch.float32, device=DEV)
    B.sq_quantize_act_tiled(up(c.x), s, xq, xs)
    odt = torch.float32 if dtype == "f32" else torch.bfloat16
    y = torch.empty((m, n), dtype=odt, device=DEV)
    bias_dev = None if c.bias is None else up(c.bias)
    B.sq_w8a8_gemm_tiled(xq, xs, m, wq, sw, n, k, bias_dev, y)
    torch.cuda.synchronize()
    s_ref, wq_ref, sw_ref = orc.prepare_weight(c.w.f32, mx, 0.5)
    xq_ref, xs_ref = orc.quantize_act(c.x.f32, s_ref)
    assert_equal(down(xs), xs_ref, "x_scale")
    assert_equal(down(B.untile(xq, m, k)), xq_ref, "x_q")
    acc = orc.int_gemm(xq_ref, wq_ref)
    bias_f = None if c.bias is None else c.bias.f32
    yref = orc.dequant(acc, xs_ref, sw_ref, bias_f)
    scale = np.abs(acc.astype(np.float64) * xs_ref[:, None] * sw_ref[None, :])
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if odt == torch.float32:
        assert_f32_rel(down(y), yref, scale)
    else:
        # the cancellation allowance only with a bias; without one the strict 1-ulp bar
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref), *(() if bias_f is None else (yref, scale)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(5, 40, 272), (70, 33, 1040), (300, 129, 528), (16, 1000, 4096)], ids=_id)
def test_layer_tiled_matches_row(orc, shape, dtype):
    """SmoothQuantLinear with tiled weights: the same smoothing factor,
    scales, codes (untiled) and outputs as the row-major layer, bit for bit,
    through calibrate -> freeze -> forward, a recompute for a new alpha, an
    empty batch and quantization_error; and the codes equal the oracle's."""
    m, n, k = shape
    c = inputs.small(m, n, k, seed=23 + m + n + k, dtype=dtype)
    bias_dev = None if c.bias is None else up(c.bias)
    layers = {lay: B.SmoothQuantLinear(up(c.w), bias_dev, alpha=0.5, layout=lay) for lay in ("row", "tiled")}
    x = up(c.x)
    for layer in layers.values():
        layer.calibrate(x[: (m + 1) // 2])
        layer.calibrate(x[(m + 1) // 2:])
        assert layer.freeze() == B.SQ_OK
    row, tiled = layers["row"], layers["tiled"]
    mx = orc.calibrate(c.x.f32)
    for alpha in (0.5, 0.25):
        if alpha != 0.5:
            for layer in layers.values():
                assert layer.recompute(alpha) == B.SQ_OK
        y_row, y_tiled = row.forward(x), tiled.forward(x)
        torch.cuda.synchronize()
        s_ref, wq_ref, sw_ref = orc.prepare_weight(c.w.f32, mx, alpha)
        assert_equal(down(tiled.smooth), s_ref, "smooth")
        assert_equal(down(tiled.weight_scale), sw_ref, "weight_scale")
        assert_equal(down(B.untile(tiled.weight_int8, n, k)), wq_ref, "weight codes")
        assert_equal(down(row.weight_int8), wq_ref, "row-major weight codes")
        assert_equal(down(y_tiled), down(y_row), f"output, alpha {alpha}")
    assert tiled.forward(x[:0]).shape == (0, n)
    assert tiled.quantization_error(x) == row.quantization_error(x)
    with pytest.raises(ValueError):
        B.SmoothQuantLinear(up(c.w), layout="columns")


# ---------------------------------------------------------------------------
# Weight-only int8 linear on tiled weights (torchao page
# "quantization/subclass.py", Int8WeightOnlyQuantizedLinearWeight). The bar
# is the row-major call's, derived from the arithmetic (exact products, an
# fp32 sum of K terms in any order within K 2^-24 sum |x w|, one rounding
# each for the scale and the bias, half a bf16 ulp for bf16 output), and the
# result equals the row-major call's bit for bit (same sums in the same
# order; the padding columns add zeros).
# ---------------------------------------------------------------------------
WO_SHAPES = [(1, 1, 16), (3, 17, 48), (16, 100, 272), (16, 200, 4096), (33, 64, 528), (64, 129, 1040),
             (80, 70, 256), (130, 40, 4112), (16, 11008, 4096), (5, 4099, 80)]


def _assert_wo_close(got, yref, mag, k, out):
    if out == "f32":
        g = got.astype(np.float64)
        half_ulp = 0.0
    else:
        g = (got.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        e = np.floor(np.log2(np.maximum(np.abs(yref), 2.0 ** -126)))
        half_ulp = 2.0 ** (e - 8)
    bound = k * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(yref) + half_ulp + 1e-30
    bad = np.abs(g - yref) > bound
    assert not bad.any(), int(bad.sum())


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", WO_SHAPES, ids=_id)
def test_wo_linear_tiled(orc, shape, out, bias):
    m, n, k = shape
    print(f"tiled weight-only {m}x{n}x{k} out={out} bias={bias}", flush=True)
    rng = np.random.default_rng(m * 3 + n * 5 + k + 1)
    c = inputs.small(m, n, k, seed=23 + m + n + k, dtype="bf16", bias=bias is not None)
    wq = _codes(rng, n, k)
    sw = (rng.random(n, dtype=np.float32) * np.float32(0.002) + np.float32(1e-4)).astype(np.float32)
    bias_f = bias_t = None
    if bias == "f32":
        bias_f, bias_t = c.bias.f32, up(c.bias.f32)
    elif bias == "bf16":
        bias_f, bias_t = c.bias.f32, up(c.bias)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y = torch.zeros((m, n), dtype=odt, device=DEV)
    x_dev = up(c.x)
    B.sq_wo_linear_tiled(x_dev, up(_tile_host(wq, rng)), up(sw), n, bias_t, y)
    y_rm = torch.zeros((m, n), dtype=odt, device=DEV)
    B.sq_wo_linear(x_dev, up(wq), up(sw), bias_t, y_rm)
    torch.cuda.synchronize()
    yref = orc.wo_linear(c.x.f32, wq, sw, bias_f)
    mag = (np.abs(c.x.f32.astype(np.float64)) @ np.abs(wq.astype(np.float64)).T) * sw[None, :].astype(np.float64)
    _assert_wo_close(down(y), yref, mag, k, out)
    assert_equal(down(y), down(y_rm), "tiled vs row-major")


def test_wo_linear_tiled_from_prepared_weights(orc):
    """The layer's route: weights prepared uncalibrated into tiles (s = 1),
    then the tiled weight-only product on the decode shape."""
    m, n, k = 16, 11008, 4096
    c = inputs.small(m, n, k, seed=5, dtype="bf16", bias=False)
    s = torch.empty(k, dtype=torch.float32, device=DEV)
    wq = B.tiled_empty(n, k, DEV)
    sw = torch.empty(n, dtype=torch.float32, device=DEV)
    assert B.sq_prepare_weight_tiled(up(c.w), None, 0.5, s, wq, sw) == B.SQ_WARN_UNCALIBRATED
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    B.sq_wo_linear_tiled(up(c.x), wq, sw, n, None, y)
    torch.cuda.synchronize()
    wq_ref, sw_ref = orc.quantize_rows(c.w.f32.copy())
    assert_equal(down(sw), sw_ref, "w_scale")
    assert_equal(down(B.untile(wq, n, k)), wq_ref, "w_q")
    yref = orc.wo_linear(c.x.f32, wq_ref, sw_ref, None)
    mag = (np.abs(c.x.f32.astype(np.float64)) @ np.abs(wq_ref.astype(np.float64)).T) * sw_ref[None, :]
    _assert_wo_close(down(y), yref, mag, k, "bf16")


# ---------------------------------------------------------------------------
# Per-tensor variant on tiled codes (page "quantized_linear.py",
# quantize_tensor and QuantizedLinear.forward): the one scale and the codes
# equal the oracle's and the row-major call's; the product equals the
# row-major per-tensor product bit for bit and the oracle to the usual bar.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (17, 80), (130, 528), (257, 1040), (1000, 4096)], ids=_id)
def test_quantize_tensor_tiled(orc, shape, dtype):
    m, k = shape
    c = inputs.small(m, 8, k, seed=13 + m + k, dtype=dtype, bias=False)
    q = _garbage(m, k)
    sc = torch.zeros(1, dtype=torch.float32, device=DEV)
    B.sq_quantize_tensor_tiled(up(c.x), q, sc)
    torch.cuda.synchronize()
    q_ref, sc_ref = orc.quantize_tensor(c.x.f32)
    assert_equal(down(sc)[0], sc_ref, "scale")
    assert_equal(down(B.untile(q, m, k)), q_ref, "codes")
    assert not _padding_columns(q, m, k).any(), "padding columns not zero"


@pytest.mark.parametrize("bias", [None, "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 5, 32), (16, 200, 4096), (64, 129, 528), (130, 260, 528),
                                   (257, 300, 1040)], ids=_id)
def test_gemm_per_tensor_tiled(orc, shape, out, bias):
    m, n, k = shape
    c = inputs.small(m, n, k, seed=5 + m + n + k, dtype="bf16", bias=bias is not None)
    x_dev, w_dev = up(c.x), up(c.w)
    xq, sx = B.tiled_empty(m, k, DEV), torch.zeros(1, dtype=torch.float32, device=DEV)
    wq, sw = B.tiled_empty(n, k, DEV), torch.zeros(1, dtype=torch.float32, device=DEV)
    B.sq_quantize_tensor_tiled(x_dev, xq, sx)
    B.sq_quantize_tensor_tiled(w_dev, wq, sw)
    bias_f = bias_t = None
    if bias == "f32":
        bias_f, bias_t = c.bias.f32, up(c.bias.f32)
    elif bias == "bf16":
        bias_f, bias_t = c.bias.f32, up(c.bias)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y = torch.zeros((m, n), dtype=odt, device=DEV)
    B.sq_w8a8_gemm_per_tensor_tiled(xq, sx, m, wq, sw, n, k, bias_t, y)
    xq_r, sx_r = torch.zeros((m, k), dtype=torch.int8, device=DEV), torch.zeros(1, dtype=torch.float32, device=DEV)
    wq_r, sw_r = torch.zeros((n, k), dtype=torch.int8, device=DEV), torch.zeros(1, dtype=torch.float32, device=DEV)
    B.sq_quantize_tensor(x_dev, xq_r, sx_r)
    B.sq_quantize_tensor(w_dev, wq_r, sw_r)
    y_rm = torch.zeros((m, n), dtype=odt, device=DEV)
    B.sq_w8a8_gemm_per_tensor(xq_r, sx_r, wq_r, sw_r, bias_t, y_rm)
    torch.cuda.synchronize()
    xq_ref, sx_ref, wq_ref, sw_ref, acc, yref = orc.linear_per_tensor(c.x.f32, c.w.f32, bias_f)
    assert_equal(down(B.untile(xq, m, k)), xq_ref, "x codes")
    assert_equal(down(B.untile(wq, n, k)), wq_ref, "w codes")
    scale = np.abs(acc.astype(np.float64) * float(sx_ref) * float(sw_ref))
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if out == "f32":
        assert_f32_rel(down(y), yref, scale)
    else:
        # the cancellation allowance only with a bias; without one the strict 1-ulp bar
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref), *(() if bias_f is None else (yref, scale)))
    assert_equal(down(y), down(y_rm), "tiled vs row-major")
