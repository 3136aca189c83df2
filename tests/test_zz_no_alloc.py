"""sq_w8a8_linear_noalloc (the activation codes in the library's fixed
device array, nothing allocated) against sq_w8a8_linear (a caller
workspace): the same output bits, on two calls in a row, the second with a
smaller input, and against the oracle's codes through sq_w8a8_linear's
workspace. Also the host-side refusals beyond the array's limits."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_equal, down, require_gpu, up
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import inputs

OK_PTR = 0x10000


def test_noalloc_limits_host():
    L = B.lib()
    f = L.sq_w8a8_linear_noalloc
    P = OK_PTR
    # beyond the fixed array: refused before any launch
    assert f(P, B.SQ_BF16, 4097, 4096, P, P, P, 64, None, P, B.SQ_BF16, None) == B.SQ_ERR_WORKSPACE
    assert f(P, B.SQ_BF16, B.SQ_NOALLOC_MAX_TOKENS + 1, 16, P, P, P, 64, None, P, B.SQ_BF16,
             None) == B.SQ_ERR_WORKSPACE
    # the linear's own checks
    assert f(P, B.SQ_I32, 4, 64, P, P, P, 8, None, P, B.SQ_BF16, None) == B.SQ_ERR_DTYPE
    assert f(P, B.SQ_BF16, 4, 40, P, P, P, 8, None, P, B.SQ_BF16, None) == B.SQ_ERR_ALIGN
    assert f(None, B.SQ_BF16, 4, 64, P, P, P, 8, None, P, B.SQ_BF16, None) == B.SQ_ERR_ARG
    assert f(P, B.SQ_BF16, 4, 64, P, P, P, 0, None, P, B.SQ_BF16, None) == B.SQ_ERR_SHAPE
    assert f(None, B.SQ_BF16, 0, 64, None, None, None, 8, None, None, B.SQ_BF16, None) == B.SQ_OK


def _prepared(orc, m, n, k, seed, dtype):
    c = inputs.small(m, n, k, seed=seed, dtype=dtype, bias=True)
    s, wq, sw = orc.prepare_weight(c.w.f32, orc.calibrate(c.x.f32), 0.5)
    return c, s, wq, sw


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_linear(orc, dtype):
    require_gpu()
    out = torch.bfloat16 if dtype == "bf16" else torch.float32
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    # first a large call (the MFMA-tile product, 4096 x 4096 codes: the whole
    # array), then a smaller one (the weight-streaming product) on the same
    # array, then the large shape again with other inputs
    for (m, n, k, seed) in ((4096, 256, 4096, 1), (48, 300, 1040, 2), (4096, 256, 4096, 3), (130, 72, 528, 4)):
        c, s, wq, sw = _prepared(orc, m, n, k, seed, dtype)
        x, s_d, wq_d, sw_d, b_d = up(c.x), up(s), up(wq), up(sw), up(c.bias)
        y_ref = torch.empty((m, n), dtype=out, device=DEV)
        ws = torch.empty(B.sq_w8a8_linear_workspace_bytes(m, k), dtype=torch.uint8, device=DEV)
        B.sq_w8a8_linear(x, s_d, wq_d, sw_d, b_d, y_ref, ws)
        y = torch.full((m, n), 7.0, dtype=out, device=DEV)
        assert B.sq_w8a8_linear_noalloc(x, s_d, wq_d, sw_d, b_d, y) == B.SQ_OK
        torch.cuda.synchronize()
        print(f"noalloc {dtype} {m}x{k}->{n}: compared", flush=True)
        assert torch.equal(y.view(ibits), y_ref.view(ibits)), (m, n, k)
        # and the workspace route's codes are the oracle's
        xq_ref, xs_ref = orc.quantize_act(c.x.f32, s)
        xq_g, xs_g = B.workspace_views(ws, m, k)
        assert_equal(down(xs_g), xs_ref, "x_scale")
        assert_equal(down(xq_g), xq_ref, "x_q")
