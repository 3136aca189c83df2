"""sq_w8a8_linear_tiled (one forward on tiled weights: activation codes into
the workspace, then the product) and sq_w8a8_linear_tiled_fused (up to 64
tokens as ONE kernel that quantises the activations itself: a few
workgroups quantise and publish one token each, the rest wait for them,
bounded, and stream the weights). Against the two separate calls
(sq_quantize_act_tiled + sq_w8a8_gemm_tiled, the same bits) and the oracle
(codes, scales, outputs), over calls in a row on one workspace, graph
replays, the forced fallback (every workgroup quantising every token
itself) and workspace reuse."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import (DEV, assert_bf16_within_one_ulp, assert_equal, assert_f32_rel, down, require_gpu,
                      up)
from w8a8_quantized_linear_sq_amd import binding as B
from w8a8_quantized_linear_sq_amd import inputs

pytestmark = pytest.mark.gpu

OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    B.lib()
    yield
    B.sq_set_fused_wait_polls(4096)


def _prep(orc, c):
    """Weights prepared on the GPU (tiled), as a frozen layer holds them."""
    mx = orc.calibrate(c.x.f32)
    s = torch.empty(c.k, dtype=torch.float32, device=DEV)
    wq = B.tiled_empty(c.n, c.k, DEV)
    ws = torch.empty(c.n, dtype=torch.float32, device=DEV)
    B.sq_prepare_weight_tiled(up(c.w), up(mx), 0.5, s, wq, ws)
    return s, wq, ws


def _two_calls(c, s, wq, ws, bias, out):
    xq = B.tiled_empty(c.m, c.k, DEV)
    xs = torch.empty(c.m, dtype=torch.float32, device=DEV)
    B.sq_quantize_act_tiled(up(c.x), s, xq, xs)
    y = torch.empty((c.m, c.n), dtype=OUT[out], device=DEV)
    B.sq_w8a8_gemm_tiled(xq, None if out == "i32" else xs, c.m, wq, None if out == "i32" else ws, c.n, c.k,
                         None if out == "i32" else bias, y)
    return y


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_oracle(orc, c, s, wq, ws, bias_f, y, wsp, fused):
    s_h = down(s)
    xq_ref, xs_ref = orc.quantize_act(c.x.f32, s_h)
    xq_t, xs_t = B.linear_tiled_views(wsp, c.m, c.k, fused)
    assert_equal(down(B.untile(xq_t, c.m, c.k)), xq_ref, "x_q (workspace)")
    assert_equal(down(xs_t), xs_ref, "x_scale (workspace)")
    wq_h, ws_h = down(B.untile(wq, c.n, c.k)), down(ws)
    acc = orc.int_gemm(xq_ref, wq_h)
    if y.dtype == torch.int32:
        assert_equal(down(y), acc, "acc")
        return
    yref = orc.dequant(acc, xs_ref, ws_h, bias_f)
    scale = np.abs(acc.astype(np.float64) * xs_ref[:, None] * ws_h[None, :])
    if bias_f is not None:
        scale = scale + np.abs(bias_f)[None, :]
    if y.dtype == torch.float32:
        assert_f32_rel(down(y), yref, scale)
    elif bias_f is None:
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref))
    else:
        assert_bf16_within_one_ulp(down(y), orc.to_bf16(yref), yref, scale)


# (m, n, k): one token; a token group and one more; 64 tokens; few weight
# rows (fewer workgroups than tokens: each quantises several); K tails of
# 16 / 48 and the longest K
SHAPES = [(1, 33, 64), (16, 11008, 4096), (17, 200, 272), (33, 16, 48), (64, 129, 4096), (5, 40, 16384),
          (48, 4099, 1040), (64, 300, 16)]


def _id(s):
    return "x".join(map(str, s))


@pytest.mark.parametrize("out", ["bf16", "f32", "i32"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_fused_matches_two_calls_and_oracle(orc, shape, dtype, out):
    m, n, k = shape
    c = inputs.small(m, n, k, seed=5 + m + n + k, dtype=dtype, bias=True)
    s, wq, ws = _prep(orc, c)
    bias = up(c.bias)
    y2 = _two_calls(c, s, wq, ws, bias, out)
    for fused in (True, False):
        wsp = B.linear_tiled_workspace(m, k, DEV, fused=fused)
        y1 = torch.full((m, n), 3, dtype=OUT[out], device=DEV)
        call = B.sq_w8a8_linear_tiled_fused if fused else B.sq_w8a8_linear_tiled
        assert call(up(c.x), s, wq, None if out == "i32" else ws, n, None if out == "i32" else bias, y1,
                    wsp) == B.SQ_OK
        torch.cuda.synchronize()
        print(f"{'one kernel' if fused else 'linear_tiled'} {m}x{k}->{n} {dtype} {out}: compared", flush=True)
        assert torch.equal(_bits(y1), _bits(y2)), "linear and the two separate calls differ"
        _check_oracle(orc, c, s, wq, ws, None if out == "i32" else c.bias.f32, y1, wsp, fused)


def test_fused_calls_in_a_row_and_forced_fallback(orc):
    """Eight calls in a row on one workspace, each with other activations
    (every call must wait for its own tokens, not a previous call's), then
    the same with the wait disabled (every workgroup quantises every token
    itself), then back."""
    m, n, k = 16, 2048, 1040
    c0 = inputs.small(m, n, k, seed=3, dtype="bf16", bias=False)
    s, wq, ws = _prep(orc, c0)
    wsp = B.linear_tiled_workspace(m, k, DEV, fused=True)
    for polls in (4096, 0, 4096):
        B.sq_set_fused_wait_polls(polls)
        before = B.linear_tiled_fallbacks(wsp)
        for i in range(8):
            ci = inputs.small(m, n, k, seed=100 + i, dtype="bf16", bias=False)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
            B.sq_w8a8_linear_tiled_fused(up(ci.x), s, wq, ws, n, None, y, wsp)
            y2 = _two_calls(ci, s, wq, ws, None, "bf16")
            torch.cuda.synchronize()
            assert torch.equal(_bits(y), _bits(y2)), (polls, i)
        fell = B.linear_tiled_fallbacks(wsp) - before
        print(f"wait polls {polls}: 8 calls in a row match, {fell} workgroups quantised the tokens themselves",
              flush=True)
        if polls == 0:
            assert fell > 0
    B.sq_set_fused_wait_polls(4096)


def test_fused_graph_replays(orc):
    """Three calls captured in one HIP graph (three activation buffers, one
    workspace), replayed four times with new activations copied in between
    replays (eager work between them): every replay's outputs equal the
    two-call path on that replay's activations."""
    m, n, k = 16, 11008, 4096
    c0 = inputs.small(m, n, k, seed=7, dtype="bf16", bias=False)
    s, wq, ws = _prep(orc, c0)
    wsp = B.linear_tiled_workspace(m, k, DEV, fused=True)
    xs = [torch.empty((m, k), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    stream = torch.cuda.Stream(DEV)
    calls = [B.prepared(B.sq_w8a8_linear_tiled_fused, xs[i], s, wq, ws, n, None, ys[i], wsp, stream)
             for i in range(3)]
    for i in range(3):
        xs[i].copy_(up(inputs.small(m, n, k, seed=200 + i, dtype="bf16", bias=False).x))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for call in calls:
            call()
    torch.cuda.synchronize()
    for rep in range(4):
        cases = [inputs.small(m, n, k, seed=300 + 10 * rep + i, dtype="bf16", bias=False) for i in range(3)]
        for i in range(3):
            xs[i].copy_(up(cases[i].x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            want = _two_calls(cases[i], s, wq, ws, None, "bf16")
            torch.cuda.synchronize()
            assert torch.equal(_bits(ys[i]), _bits(want)), (rep, i)
        print(f"graph replay {rep}: 3 calls match", flush=True)


def test_fused_workspace_reuse_and_many_tokens(orc):
    """One workspace (sized for the largest call) used for 16, 1, 64, 16
    tokens in turn by the one-kernel path (its synchronisation words sit at
    a fixed place whatever m), and for up to 200 tokens by the two-launch
    linear; all equal the two separate calls. Beyond 64 tokens the
    one-kernel path refuses."""
    n, k = 300, 528
    wsp = B.linear_tiled_workspace(200, k, DEV, fused=True)
    c0 = inputs.small(200, n, k, seed=9, dtype="f32", bias=True)
    s, wq, ws = _prep(orc, c0)
    for m in (16, 1, 64, 65, 200, 16):
        c = inputs.small(m, n, k, seed=400 + m, dtype="f32", bias=True)
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        if m <= 64:
            B.sq_w8a8_linear_tiled_fused(up(c.x), s, wq, ws, n, up(c.bias), y, wsp)
        else:
            with pytest.raises(B.SQError):
                B.sq_w8a8_linear_tiled_fused(up(c.x), s, wq, ws, n, up(c.bias), y, wsp)
            B.sq_w8a8_linear_tiled(up(c.x), s, wq, ws, n, up(c.bias), y, wsp)
        y2 = _two_calls(c, s, wq, ws, up(c.bias), "f32")
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y2)), m
