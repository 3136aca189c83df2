"""The ragged grid M, N in {1..7, 17, 33} x K in {16, 32, 48, 272}, every
shape through the whole path (running max, weight preparation, activation
codes, the product with a bias and fp32 out), row-major and in 16 x 64 tiles,
against the oracle: the running max, s, both sides' int8 codes and scales
bit for bit; outputs within 1e-6 of |acc sx sw| + |bias|. Odd M + N take
fp32 inputs, even ones bf16."""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_equal, assert_f32_rel, down, require_gpu, up
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import inputs

pytestmark = pytest.mark.gpu

MN = [1, 2, 3, 4, 5, 6, 7, 17, 33]
KS = [16, 32, 48, 272]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    B.lib()


def _zeros(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device=DEV)


@pytest.mark.parametrize("layout", ["row", "tiled"])
@pytest.mark.parametrize("k", KS)
def test_ragged_grid(orc, k, layout):
    for m, n in itertools.product(MN, MN):
        what = f"{m}x{n}x{k} {layout}"
        c = inputs.small(m, n, k, seed=1000 + 37 * m + 11 * n + k, dtype="f32" if (m + n) % 2 else "bf16",
                         bias=True)
        x, w, b = up(c.x), up(c.w), up(c.bias)
        run = _zeros(k, torch.float32)
        B.sq_calibrate(x, run)
        s = _zeros(k, torch.float32)
        sw = _zeros(n, torch.float32)
        y = _zeros((m, n), torch.float32)
        if layout == "row":
            wq = _zeros((n, k), torch.int8)
            B.sq_prepare_weight(w, run, 0.5, s, wq, sw)
            wsp = torch.empty(B.sq_w8a8_linear_workspace_bytes(m, k), dtype=torch.uint8, device=DEV)
            B.sq_w8a8_linear(x, s, wq, sw, b, y, wsp)
            xq, xs = B.workspace_views(wsp, m, k)
        else:
            wq = B.tiled_empty(n, k, DEV)
            B.sq_prepare_weight_tiled(w, run, 0.5, s, wq, sw)
            xq = B.tiled_empty(m, k, DEV)
            xs = _zeros(m, torch.float32)
            B.sq_quantize_act_tiled(x, s, xq, xs)
            B.sq_w8a8_gemm_tiled(xq, xs, m, wq, sw, n, k, b, y)
            xq, wq = B.untile(xq, m, k), B.untile(wq, n, k)
        torch.cuda.synchronize()
        mx = orc.calibrate(c.x.f32)
        s_r, wq_r, sw_r = orc.prepare_weight(c.w.f32, mx, 0.5)
        xq_r, xs_r, acc, y_r = orc.linear(c.x.f32, s_r, wq_r, sw_r, c.bias.f32)
        assert_equal(down(run), mx, f"{what}: running max")
        assert_equal(down(s), s_r, f"{what}: s")
        assert_equal(down(wq), wq_r, f"{what}: w_q")
        assert_equal(down(sw), sw_r, f"{what}: w_scale")
        assert_equal(down(xq), xq_r, f"{what}: x_q")
        assert_equal(down(xs), xs_r, f"{what}: x_scale")
        scale = np.abs(acc.astype(np.float64) * xs_r[:, None] * sw_r[None, :]) + np.abs(c.bias.f32)[None, :]
        assert_f32_rel(down(y), y_r, scale)
