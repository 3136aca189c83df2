"""Helpers shared by the GPU parity tests: uploads and comparisons."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible")


def up(t, dtype: str | None = None) -> torch.Tensor:
    """Upload an inputs.Tensor (bf16 bits or fp32) or a numpy array."""
    if hasattr(t, "f32"):
        if t.bits is not None:
            return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(DEV).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(t.f32)).to(DEV)
    a = np.ascontiguousarray(t)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def down(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_bf16_within_one_ulp(got_bits: np.ndarray, want_bits: np.ndarray, yref: np.ndarray | None = None,
                               scale: np.ndarray | None = None, rel: float = 1e-6):
    """bf16 outputs within 1 ulp (ordinal distance) of the oracle's value
    rounded once. Where a bias cancels the product the result is small and
    its fp32 rounding error is not small against a bf16 ulp of it; there
    (``yref``/``scale`` given) the bar is |got - yref| <= rel * scale + half
    a bf16 ulp of got, scale = |acc sx sw| + |bias|."""
    d = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(want_bits))
    bad = d > 1
    if yref is not None and bad.any():
        g = _bf16_values(got_bits[bad])
        # g = f * 2^e with f in [0.5, 1): a bf16 ulp there is 2^(e - 8)
        half_ulp = np.ldexp(1.0, np.frexp(np.where(g == 0, 1e-38, g))[1] - 9)
        ok = np.abs(g - yref[bad]) <= rel * scale[bad] + half_ulp
        bad_idx = np.argwhere(bad)[~ok]
    else:
        bad_idx = np.argwhere(bad)
    assert bad_idx.size == 0, f"{len(bad_idx)} bf16 outputs beyond 1 ulp, first at {bad_idx[:3].tolist()}"


def assert_f32_rel(got: np.ndarray, want: np.ndarray, scale: np.ndarray, rel: float = 1e-6):
    """|got - want| <= rel * scale, elementwise (scale = |acc sx sw| + |bias|)."""
    err = np.abs(got.astype(np.float64) - want)
    bad = np.argwhere(err > rel * scale)
    assert bad.size == 0, f"{len(bad)} fp32 outputs beyond {rel} relative, first at {bad[:3].tolist()}"


def assert_equal(got: np.ndarray, want: np.ndarray, what: str):
    if got.dtype == np.float32 and want.dtype == np.float32:
        g, w = got.view(np.uint32), want.view(np.uint32)
    else:
        g, w = got, want
    if not np.array_equal(g, w):
        diff = np.argwhere(g != w)
        first = tuple(diff[0])
        raise AssertionError(f"{what}: {len(diff)} mismatches, first at {first}: got {got[first]!r} "
                             f"want {want[first]!r}")
