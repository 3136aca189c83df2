"""GPU parity at the workloads' full sizes, the path run as the benchmark
runs it: the running max over the calibration batches (sq_calibrate), the
smoothing factor and int8 weights (sq_prepare_weight), then the activation
codes (sq_quantize_act) and the int8 product with its dequantisation
(sq_w8a8_gemm), or the last two in one call (sq_w8a8_linear).

The same path runs on codes in 16 x 64 tiles (the _tiled calls), as the
benchmark runs it. Every maximum, smoothing factor, scale and int8 code is
compared with the oracle in full, bit for bit. Outputs are compared in full
where the oracle's integer product takes seconds (tiny, prefill, decode,
the block linears on tiles), else on seeded row samples that always include
the first and last token (block linears row-major: 96 rows; MLP
up-projection: 512 of 8192 rows, 1/16): fp32 within 1e-6 of
|acc sx sw| + |bias|, bf16 within one bf16 ulp of the oracle's binary64
result rounded once (with the bias cancellation allowance where a bias is
added). The int32 product at 4096^3 is also compared in full with the
vendor library's int8 GEMM."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_bf16_within_one_ulp, assert_equal, assert_f32_rel, down, require_gpu, up
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    B.lib()


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=DEV)


def _calibrate(case):
    """The running max as the benchmark takes it: every calibration batch
    in one sq_calibrate_batches call that starts the max (8 at most)."""
    assert len(case.calib) <= B.SQ_MAX_CALIB_BATCHES
    run = torch.full((case.k,), 1e30, dtype=torch.float32, device=DEV)
    B.sq_calibrate_batches([up(cb) for cb in case.calib], run, first=True)
    return run


def _prepare(w_dev, run, alpha, n, k):
    s = _empty(k, torch.float32)
    wq = _empty((n, k), torch.int8)
    sw = _empty(n, torch.float32)
    B.sq_prepare_weight(w_dev, run, alpha, s, wq, sw)
    return s, wq, sw


def _rows(m, count, seed):
    if count is None or count >= m:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, m - 1), size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, m - 1], mid]))


def _check_y(orc, y_dev, xq_ref, xs_ref, wq_ref, sw_ref, bias_f, rows):
    acc = orc.int_gemm(np.ascontiguousarray(xq_ref[rows]), wq_ref)
    yref = orc.dequant(acc, xs_ref[rows], sw_ref, bias_f)
    got = down(y_dev[torch.from_numpy(rows).to(DEV)])
    scale = np.abs(acc.astype(np.float64) * xs_ref[rows][:, None] * sw_ref[None, :])
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if y_dev.dtype == torch.float32:
        assert_f32_rel(got, yref, scale)
    elif bias_f is None:
        assert_bf16_within_one_ulp(got, orc.to_bf16(yref))
    else:
        assert_bf16_within_one_ulp(got, orc.to_bf16(yref), yref, scale)


def _run_and_check(orc, case, alphas, sample_rows, out_dtype, fused=False, tiled=False):
    m, n, k = case.m, case.n, case.k
    print(f"config {case.name}: m={m} n={n} k={k} alphas={alphas} fused={fused} tiled={tiled}", flush=True)
    x_dev, w_dev = up(case.x), up(case.w)
    bias_dev = None if case.bias is None else up(case.bias)
    bias_f = None if case.bias is None else case.bias.f32

    run = _calibrate(case)
    torch.cuda.synchronize()
    run_ref = np.zeros(k, np.float32)
    for cb in case.calib:
        orc.calibrate(cb.f32, run_ref)
    assert_equal(down(run), run_ref, "running max")

    rows = _rows(m, sample_rows, seed=m + n + k)
    for alpha in alphas:
        if tiled:
            s, wq, sw = _empty(k, torch.float32), B.tiled_empty(n, k, DEV), _empty(n, torch.float32)
            B.sq_prepare_weight_tiled(w_dev, run, alpha, s, wq, sw)
        else:
            s, wq, sw = _prepare(w_dev, run, alpha, n, k)
        y = _empty((m, n), out_dtype)
        if tiled:
            xq, xs = B.tiled_empty(m, k, DEV), _empty(m, torch.float32)
            B.sq_quantize_act_tiled(x_dev, s, xq, xs)
            B.sq_w8a8_gemm_tiled(xq, xs, m, wq, sw, n, k, bias_dev, y)
        elif fused:
            ws = _empty(B.sq_w8a8_linear_workspace_bytes(m, k), torch.uint8)
            B.sq_w8a8_linear(x_dev, s, wq, sw, bias_dev, y, ws)
            xq, xs = B.workspace_views(ws, m, k)
        else:
            xq, xs = _empty((m, k), torch.int8), _empty(m, torch.float32)
            B.sq_quantize_act(x_dev, s, xq, xs)
            B.sq_w8a8_gemm(xq, xs, wq, sw, bias_dev, y)
        torch.cuda.synchronize()
        if tiled:
            wq, xq = B.untile(wq, n, k), B.untile(xq, m, k)

        s_ref, wq_ref, sw_ref = orc.prepare_weight(case.w.f32, run_ref, alpha)
        assert_equal(down(s), s_ref, f"smooth (alpha {alpha})")
        assert_equal(down(sw), sw_ref, f"w_scale (alpha {alpha})")
        assert_equal(down(wq), wq_ref, f"w_q (alpha {alpha})")
        xq_ref, xs_ref = orc.quantize_act(case.x.f32, s_ref)
        assert_equal(down(xs), xs_ref, f"x_scale (alpha {alpha})")
        assert_equal(down(xq), xq_ref, f"x_q (alpha {alpha})")
        _check_y(orc, y, xq_ref, xs_ref, wq_ref, sw_ref, bias_f, rows)
        del s, wq, sw, y, xq, xs


def test_tiny_f32(orc):
    _run_and_check(orc, inputs.tiny(), (0.5,), None, torch.float32)


def test_prefill_2048x4096x4096(orc):
    _run_and_check(orc, inputs.prefill(), (0.5,), None, torch.bfloat16)


def test_decode_16x4096x11008(orc):
    # the per-call path: activation codes and the product in one call
    _run_and_check(orc, inputs.decode(), (0.5,), None, torch.bfloat16, fused=True)


@pytest.mark.parametrize("layer", range(len(inputs.BLOCK_LINEARS)),
                         ids=[f"{nm}_{n}x{k}" for nm, n, k in inputs.BLOCK_LINEARS])
def test_block_linear(orc, layer):
    _run_and_check(orc, inputs.block_linear(layer), (0.5,), 96, torch.bfloat16)


@pytest.mark.parametrize("layer", range(len(inputs.BLOCK_LINEARS)),
                         ids=[f"{nm}_{n}x{k}" for nm, n, k in inputs.BLOCK_LINEARS])
def test_block_linear_tiled(orc, layer):
    """The same layers with the int8 codes in 16 x 64 tiles, as the benchmark
    runs them: every output row checked."""
    _run_and_check(orc, inputs.block_linear(layer), (0.5,), None, torch.bfloat16, tiled=True)


def test_prefill_2048x4096x4096_tiled(orc):
    _run_and_check(orc, inputs.prefill(), (0.5,), None, torch.bfloat16, tiled=True)


def test_mlp_up_8192x8192x28672_tiled(orc):
    """The MLP up-projection (with its bias) on tiled codes, alpha 0.5."""
    _run_and_check(orc, inputs.mlp_up(), (0.5,), 512, torch.bfloat16, tiled=True)


def test_mlp_up_8192x8192x28672_alpha_sweep(orc):
    case = inputs.mlp_up()
    _run_and_check(orc, case, case.alphas, 512, torch.bfloat16)


@pytest.mark.parametrize("tiled", [False, True], ids=["row", "tiled"])
def test_per_tensor_o_proj_4096(orc, tiled):
    """The per-tensor variant (page "quantized_linear.py") at the O
    projection's size: codes and scales of X and W in full, the output on
    sampled rows; row-major codes, or tiled as the benchmark runs it."""
    case = inputs.o_proj()
    m, n, k = case.m, case.n, case.k
    print(f"per-tensor {case.name} tiled={tiled}", flush=True)
    sx, sw = _empty(1, torch.float32), _empty(1, torch.float32)
    y = _empty((m, n), torch.bfloat16)
    if tiled:
        xq, wq = B.tiled_empty(m, k, DEV), B.tiled_empty(n, k, DEV)
        B.sq_quantize_tensor_tiled(up(case.x), xq, sx)
        B.sq_quantize_tensor_tiled(up(case.w), wq, sw)
        B.sq_w8a8_gemm_per_tensor_tiled(xq, sx, m, wq, sw, n, k, None, y)
        torch.cuda.synchronize()
        xq, wq = B.untile(xq, m, k), B.untile(wq, n, k)
    else:
        xq, wq = _empty((m, k), torch.int8), _empty((n, k), torch.int8)
        B.sq_quantize_tensor(up(case.x), xq, sx)
        B.sq_quantize_tensor(up(case.w), wq, sw)
        B.sq_w8a8_gemm_per_tensor(xq, sx, wq, sw, None, y)
        torch.cuda.synchronize()
    xq_ref, sx_ref = orc.quantize_tensor(case.x.f32)
    wq_ref, sw_ref = orc.quantize_tensor(case.w.f32)
    assert_equal(down(sx)[0], sx_ref, "x scale")
    assert_equal(down(sw)[0], sw_ref, "w scale")
    assert_equal(down(xq), xq_ref, "x codes")
    assert_equal(down(wq), wq_ref, "w codes")
    rows = _rows(m, 64, seed=17)
    _check_y(orc, y, xq_ref, np.full(m, sx_ref, np.float32), wq_ref, np.full(n, sw_ref, np.float32), None, rows)


def _wo_case(orc, case, sample_rows):
    """Weight-only int8 linear (torchao page "quantization/subclass.py") on
    a full-size case: plain per-channel int8 weights (sq_prepare_weight never
    calibrated, s = 1), compared bit for bit; the bf16 output on sampled rows
    against the oracle's binary64 result, within the fp32 summation bound
    K 2^-24 sum|x w| sw plus the scale and bias roundings and half a bf16 ulp."""
    m, n, k = case.m, case.n, case.k
    print(f"weight-only {case.name}", flush=True)
    s, wq, sw = _empty(k, torch.float32), _empty((n, k), torch.int8), _empty(n, torch.float32)
    assert B.sq_prepare_weight(up(case.w), None, 0.5, s, wq, sw) == B.SQ_WARN_UNCALIBRATED
    bias_dev = None if case.bias is None else up(case.bias)
    bias_f = None if case.bias is None else case.bias.f32
    y = _empty((m, n), torch.bfloat16)
    B.sq_wo_linear(up(case.x), wq, sw, bias_dev, y)
    torch.cuda.synchronize()
    s_ref, wq_ref, sw_ref = orc.prepare_weight(case.w.f32, None, 0.5)
    assert (s_ref == 1.0).all()
    assert_equal(down(s), s_ref, "smooth")
    assert_equal(down(sw), sw_ref, "w_scale")
    assert_equal(down(wq), wq_ref, "w_q")
    rows = _rows(m, sample_rows, seed=m + 7 * n)
    x_rows = np.ascontiguousarray(case.x.f32[rows])
    yref = orc.wo_linear(x_rows, wq_ref, sw_ref, bias_f)
    mag = (np.abs(x_rows.astype(np.float64)) @ np.abs(wq_ref.astype(np.float64)).T) * sw_ref[None, :]
    if bias_f is not None:
        mag = mag + np.abs(bias_f)[None, :]
    got = down(y[torch.from_numpy(rows).to(DEV)])
    got = (got.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(yref), 2.0 ** -126)))
    bound = k * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(yref) + 2.0 ** (e - 8)
    err = np.abs(got - yref)
    assert (err <= bound).all(), (int((err > bound).sum()), float((err / bound).max()))


def test_weight_only_decode_16x4096x11008(orc):
    _wo_case(orc, inputs.decode(), None)


def test_weight_only_prefill_2048x4096x4096(orc):
    _wo_case(orc, inputs.prefill(), 64)


def test_mlp_up_alpha_sweep_quantization_error(orc):
    """quantization_error across the MLP up-projection's alpha sweep (page
    "w8a8_smoothquant.py": recompute_smooth_scale from the stored maxima, then
    quantization_error): the stored weight column max and every alpha's s,
    codes and scales bit for bit; the reference linear and the quantized
    output (fp32) on sampled rows; the error reduction against the oracle's
    on the full outputs, within the binary64 summation bound."""
    case = inputs.mlp_up()
    m, n, k = case.m, case.n, case.k
    print(f"alpha sweep {case.name}", flush=True)
    x_dev, w_dev, b_dev = up(case.x), up(case.w), up(case.bias)
    run = _calibrate(case)
    mw = _empty(k, torch.float32)
    B.sq_weight_col_max(w_dev, mw)
    y_fp = _empty((m, n), torch.float32)
    B.sq_reference_linear(x_dev, w_dev, b_dev, y_fp)
    torch.cuda.synchronize()
    run_ref = np.zeros(k, np.float32)
    for cb in case.calib:
        orc.calibrate(cb.f32, run_ref)
    assert_equal(down(mw), orc.weight_col_max(case.w.f32), "weight column max")

    rows = _rows(m, 12, seed=99)
    x_rows = np.ascontiguousarray(case.x.f32[rows])
    yfp_ref = orc.reference_linear(x_rows, case.w.f32, case.bias.f32)
    mag = np.abs(x_rows.astype(np.float64)) @ np.abs(case.w.f32.astype(np.float64)).T
    got = down(y_fp[torch.from_numpy(rows).to(DEV)]).astype(np.float64)
    bound = k * 2.0 ** -24 * mag + 2.0 ** -23 * np.abs(yfp_ref)
    assert (np.abs(got - yfp_ref) <= bound).all()
    y_fp_host = down(y_fp).astype(np.float64)

    s, wq, sw = _empty(k, torch.float32), _empty((n, k), torch.int8), _empty(n, torch.float32)
    xq, xs = _empty((m, k), torch.int8), _empty(m, torch.float32)
    y_q = _empty((m, n), torch.float32)
    ws = _empty(B.sq_relative_error_workspace_bytes(m * n), torch.uint8)
    res = _empty(3, torch.float64)
    errors = {}
    for alpha in (*case.alphas, None):
        st = B.sq_recompute_smooth_scale(w_dev, None if alpha is None else run, mw, 0.5 if alpha is None else alpha,
                                         s, wq, sw)
        assert st == (B.SQ_WARN_UNCALIBRATED if alpha is None else B.SQ_OK)
        B.sq_quantize_act(x_dev, s, xq, xs)
        B.sq_w8a8_gemm(xq, xs, wq, sw, b_dev, y_q)
        B.sq_relative_error(y_fp, y_q, ws, res)
        torch.cuda.synchronize()
        s_ref, wq_ref, sw_ref = orc.prepare_weight(case.w.f32, None if alpha is None else run_ref,
                                                   0.5 if alpha is None else alpha)
        assert_equal(down(s), s_ref, f"smooth (alpha {alpha})")
        assert_equal(down(sw), sw_ref, f"w_scale (alpha {alpha})")
        assert_equal(down(wq), wq_ref, f"w_q (alpha {alpha})")
        xq_ref, xs_ref = orc.quantize_act(case.x.f32, s_ref)
        assert_equal(down(xs), xs_ref, f"x_scale (alpha {alpha})")
        _check_y(orc, y_q, xq_ref, xs_ref, wq_ref, sw_ref, case.bias.f32, rows)
        got = down(res)
        ratio, num, den = orc.relative_error(y_fp_host, down(y_q))
        tol = (m * n + 64) * 2.0 ** -53
        assert abs(got[0] - num) <= tol * num and abs(got[1] - den) <= tol * den
        assert abs(got[2] - ratio) <= 2 * tol * ratio
        errors[alpha] = float(got[2])
        print(f"alpha {alpha}: quantization_error {got[2]:.6g}", flush=True)
    # smoothing helps on outlier channels (x100 on 0.5% of them)
    assert errors[0.5] < errors[None], errors


@pytest.mark.parametrize("tiled", [False, True], ids=["row", "tiled"])
def test_int32_product_matches_vendor_library_4096(tiled):
    """The exact int32 product at M = N = K = 4096 on the O projection's
    codes, every element, against the vendor library's int8 GEMM
    (torch._int_mm): two exact integer products must agree bit for bit. The
    oracle checks these codes and sampled rows of the product; this covers
    all 16.8M outputs."""
    case = inputs.o_proj()
    m, n, k = case.m, case.n, case.k
    run = _calibrate(case)
    s, sx, sw = _empty(k, torch.float32), _empty(m, torch.float32), _empty(n, torch.float32)
    y = _empty((m, n), torch.int32)
    if tiled:
        xq, wq = B.tiled_empty(m, k, DEV), B.tiled_empty(n, k, DEV)
        B.sq_prepare_weight_tiled(up(case.w), run, 0.5, s, wq, sw)
        B.sq_quantize_act_tiled(up(case.x), s, xq, sx)
        B.sq_w8a8_gemm_tiled(xq, None, m, wq, None, n, k, None, y)
        xr, wr = B.untile(xq, m, k), B.untile(wq, n, k)
    else:
        xr, wr = _empty((m, k), torch.int8), _empty((n, k), torch.int8)
        B.sq_prepare_weight(up(case.w), run, 0.5, s, wr, sw)
        B.sq_quantize_act(up(case.x), s, xr, sx)
        B.sq_w8a8_gemm(xr, None, wr, None, None, y)
    ref = torch._int_mm(xr, wr.t())  # (k x n): the transposed view of W_q
    torch.cuda.synchronize()
    assert torch.equal(y, ref), int((y != ref).sum())


VENDOR_CASES = {"prefill": inputs.prefill, "qkv": lambda: inputs.block_linear(0), "up": lambda: inputs.block_linear(2),
                "down": lambda: inputs.block_linear(3), "mlp_up": inputs.mlp_up}


@pytest.mark.parametrize("name", list(VENDOR_CASES))
def test_int32_product_matches_vendor_library_full_size(name):
    """The exact int32 product of every other full-size workload (tiled
    codes, alpha 0.5), every element, against the vendor library's int8
    GEMM on the same codes (untiled): where the output checks against the
    oracle are sampled (the MLP up-projection: 1 row in 16), this covers
    every accumulator, including the 8192 x 28672 ones."""
    case = VENDOR_CASES[name]()
    m, n, k = case.m, case.n, case.k
    print(f"[{name}] {m}x{n}x{k}", flush=True)
    run = _calibrate(case)
    s, sx, sw = _empty(k, torch.float32), _empty(m, torch.float32), _empty(n, torch.float32)
    xq, wq = B.tiled_empty(m, k, DEV), B.tiled_empty(n, k, DEV)
    B.sq_prepare_weight_tiled(up(case.w), run, 0.5, s, wq, sw)
    B.sq_quantize_act_tiled(up(case.x), s, xq, sx)
    y = _empty((m, n), torch.int32)
    B.sq_w8a8_gemm_tiled(xq, None, m, wq, None, n, k, None, y)
    ref = torch._int_mm(B.untile(xq, m, k), B.untile(wq, n, k).t())
    torch.cuda.synchronize()
    assert torch.equal(y, ref), int((y != ref).sum())
