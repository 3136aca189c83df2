"""Seeded synthetic inputs for the SmoothQuant W8A8 linear.

This module holds no step of the method: it only draws activations, weights,
biases and calibration rows, with per-channel outliers, and rounds them to the
storage type. Both the GPU tests/bench and the CPU oracle are fed from it.

Recipe (all draws with numpy ``default_rng`` / PCG64):
  * standard normals drawn in float32, multiplied by sigma (float32);
  * a set of outlier input channels, chosen without replacement, whose
    activation columns are multiplied by a factor (x40, x50 or x100);
  * for bf16 workloads every tensor is then rounded to bf16
    (round-to-nearest-even on the float32 bit pattern); the float32 view of
    those bf16 values is exact and is what the oracle reads.
The five workloads mirror the ones the method is measured on: a tiny fp32
layer, a 2048-token prefill, a 16-token decode against an 11008x4096 weight,
a large 8192x8192 -> 28672 MLP up-projection with an alpha sweep, and one
transformer block's four linears at 4096 tokens with a separate 512-token
calibration set.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """One input tensor: its float32 values and, for bf16 storage, its bits."""
    f32: np.ndarray
    bits: np.ndarray | None = None  # uint16 bf16 patterns when dtype is bf16

    @property
    def shape(self):
        return self.f32.shape


def _store(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(x, np.float32))
    if dtype == "bf16":
        b = bf16_bits(x)
        return Tensor(bf16_to_f32(b), b)
    raise ValueError(dtype)


@dataclass
class LinearCase:
    """One linear layer's workload."""
    name: str
    dtype: str                      # storage/compute input type: "f32" or "bf16"
    x: Tensor                       # M x K activations
    w: Tensor                       # N x K weight (nn.Linear layout)
    bias: Tensor | None             # N, or None
    calib: list = field(default_factory=list)  # list of Tensor (R_i x K) batches
    alphas: tuple = (0.5,)
    outliers: np.ndarray | None = None

    @property
    def m(self):
        return self.x.shape[0]

    @property
    def k(self):
        return self.x.shape[1]

    @property
    def n(self):
        return self.w.shape[0]


def _normal(rng, shape, sigma):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def _acts(rng, m, k, chans, mult):
    x = rng.standard_normal((m, k), dtype=np.float32)
    if chans is not None and len(chans):
        x[:, chans] *= np.float32(mult)
    return x


def outlier_channels(seed: int, k: int, frac: float) -> np.ndarray:
    """round(frac * k) distinct channels, sorted."""
    cnt = int(round(frac * k))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(k, size=cnt, replace=False))


def tiny() -> LinearCase:
    """16x256 fp32 activations with channels {3, 77, 200} x40, W 128x256
    N(0, 0.02), bias N(0, 0.01), alpha 0.5; one generator, seed 0, drawing
    X, W, bias in that order; calibrated on the same 16 tokens."""
    rng = np.random.default_rng(0)
    chans = np.array([3, 77, 200])
    x = _acts(rng, 16, 256, chans, 40.0)
    w = _normal(rng, (128, 256), 0.02)
    b = _normal(rng, (128,), 0.01)
    xt = _store(x, "f32")
    return LinearCase("tiny_16x256x128_f32", "f32", xt, _store(w, "f32"), _store(b, "f32"),
                      [xt], (0.5,), chans)


def synthetic(name, m, n, k, *, seed_base, dtype="bf16", out_frac=0.01, out_mult=50.0,
              w_sigma=0.02, bias_sigma=None, alphas=(0.5,), calib_rows=None,
              calib_batches=1) -> LinearCase:
    """A general outlier-channel linear. Seeds: X = base+1, W = base+2,
    bias = base+3, outlier set = base+4, calibration = base+5. With
    ``calib_rows`` None the layer is calibrated on its own activations,
    else on ``calib_rows`` separate tokens (same outlier set), split into
    ``calib_batches`` equal batches."""
    chans = outlier_channels(seed_base + 4, k, out_frac)
    x = _acts(np.random.default_rng(seed_base + 1), m, k, chans, out_mult)
    w = _normal(np.random.default_rng(seed_base + 2), (n, k), w_sigma)
    b = None if bias_sigma is None else _normal(np.random.default_rng(seed_base + 3), (n,), bias_sigma)
    xt = _store(x, dtype)
    if calib_rows is None:
        calib = [xt]
    else:
        c = _acts(np.random.default_rng(seed_base + 5), calib_rows, k, chans, out_mult)
        per = calib_rows // calib_batches
        calib = [_store(c[i * per:(i + 1) * per], dtype) for i in range(calib_batches)]
    return LinearCase(name, dtype, xt, _store(w, dtype), None if b is None else _store(b, dtype),
                      calib, tuple(alphas), chans)


def prefill() -> LinearCase:
    """2048x4096 bf16, 1% channels x50, W 4096x4096 N(0, 0.02), no bias,
    alpha 0.5, calibrated on the same 2048 tokens."""
    return synthetic("prefill_2048x4096x4096_bf16", 2048, 4096, 4096, seed_base=2000)


def decode() -> LinearCase:
    """16x4096 bf16, 1% channels x50, W 11008x4096 N(0, 0.02), alpha 0.5."""
    return synthetic("decode_16x4096x11008_bf16", 16, 11008, 4096, seed_base=3000)


def mlp_up() -> LinearCase:
    """8192x8192 bf16, 0.5% channels x100, W 28672x8192 N(0, 0.015), bias
    N(0, 0.01), alpha swept over {0.25, 0.5, 0.75}."""
    return synthetic("mlp_up_8192x8192x28672_bf16", 8192, 28672, 8192, seed_base=4000,
                     out_frac=0.005, out_mult=100.0, w_sigma=0.015, bias_sigma=0.01,
                     alphas=(0.25, 0.5, 0.75))


# One transformer block's four linears at 4096 tokens: (name, N, K).
BLOCK_LINEARS = (("qkv", 12288, 4096), ("o", 4096, 4096), ("up", 11008, 4096),
                 ("down", 4096, 11008))


def block_linear(layer: int) -> LinearCase:
    """Layer ``layer`` (0 qkv, 1 o, 2 up, 3 down) of the block: M = 4096,
    1% channels x50, W N(0, 0.02), no bias, alpha 0.5, calibrated by a
    running max over 512 separate tokens fed as 4 batches of 128."""
    nm, n, k = BLOCK_LINEARS[layer]
    return synthetic(f"block_{nm}_4096x{k}x{n}_bf16", 4096, n, k, seed_base=5000 + 100 * layer,
                     calib_rows=512, calib_batches=4)


def o_proj() -> LinearCase:
    """The block's O projection, M = N = K = 4096 (the headline shape)."""
    return block_linear(1)


def upstream_grad(m, n, *, seed, dtype="bf16") -> Tensor:
    """An upstream gradient dL/dY for the backward: m x n standard normals
    drawn in float32 (seed ``seed``), stored as ``dtype``."""
    return _store(np.random.default_rng(seed).standard_normal((m, n), dtype=np.float32), dtype)


def small(m, n, k, *, seed=7, dtype="bf16", bias=True, out_frac=0.01, out_mult=50.0,
          calib_rows=None, calib_batches=1) -> LinearCase:
    """A small case of the same structure for parity tests (ragged sizes)."""
    out_frac = max(out_frac, 1.0 / k)  # at least one outlier channel
    return synthetic(f"small_{m}x{k}x{n}_{dtype}", m, n, k, seed_base=10000 + seed, dtype=dtype,
                     out_frac=out_frac, out_mult=out_mult, bias_sigma=0.01 if bias else None,
                     calib_rows=calib_rows, calib_batches=calib_batches)
