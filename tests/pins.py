"""Pins of the CPU oracle against what the page and mathematics fix.

Each pin is a function of an ``oracle.Oracle`` instance that raises
AssertionError on a mismatch. ``test_oracle_pins.py`` runs them on the
oracle as built; ``test_oracle_mutants.py`` runs them on copies of the oracle
with one deliberate mistake planted, and requires every such copy to fail at
least one pin.

Source of the method: page "w8a8_smoothquant.py" (BiGRU_T_version): module
docstring (the transform, the choice of s and its alpha limits, the error
bound), calibrate_smoothquant, quantize_per_channel_symmetric,
quantize_per_token_symmetric, SmoothQuantW8A8.calibrate /
freeze_quantization / forward / quantization_error.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from exact import (FLOOR, bf16_bits_of, rn_bf16, rn_f32, rn_f32_pow,
                   rn_f32_root, round_half_even)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _outlier_acts(rng, m, k, chans=(1,), mult=40.0):
    x = rng.standard_normal((m, k), dtype=np.float32)
    x[:, list(chans)] *= np.float32(mult)
    return x


def _with_ties(rng, m, k):
    """Rows whose max is 127 * 2^e so that scale = 2^e exactly and several
    entries sit exactly on half-integers after division by the scale."""
    e = rng.integers(-8, 4, size=m)
    x = np.empty((m, k), np.float32)
    for r in range(m):
        codes = rng.integers(-126, 127, size=k).astype(np.float64)
        halves = rng.random(k) < 0.5
        codes[halves] += 0.5 * np.sign(rng.standard_normal(halves.sum()))
        codes = np.clip(codes, -126.5, 126.5)
        codes[rng.integers(k)] = 127.0 * (1 if rng.random() < 0.5 else -1)
        x[r] = (codes * 2.0 ** float(e[r])).astype(np.float32)
    return x


# ---------------------------------------------------------------------------
# 1. Hand-derived worked example (tests/golden/hand_worked_alpha_half.json).
# ---------------------------------------------------------------------------
def pin_golden_hand_example(o):
    d = json.load(open(os.path.join(GOLDEN, "hand_worked_alpha_half.json")))
    x = np.array(d["x"], np.float32)
    w = np.array(d["w"], np.float32)
    b = np.array(d["bias"], np.float32)
    ex = {kk: np.array(v) for kk, v in d["expected"].items()}
    mx = o.calibrate(x)
    assert np.array_equal(mx, ex["mx"].astype(np.float32)), mx
    mw = o.weight_col_max(w)
    assert np.array_equal(mw, ex["mw"].astype(np.float32)), mw
    s = o.smoothing_factor(mx, mw, d["alpha"])
    assert np.array_equal(s, ex["s"].astype(np.float32)), s
    xs = o.smooth_act(x, s)
    assert np.array_equal(xs, ex["x_smooth"].astype(np.float32))
    ws = o.smooth_weight(w, s)
    assert np.array_equal(ws, ex["w_smooth"].astype(np.float32))
    xq, sx = o.quantize_rows(xs)
    assert np.array_equal(sx, ex["scale_x"].astype(np.float32))
    assert np.array_equal(xq, ex["xq"].astype(np.int8)), xq
    wq, sw = o.quantize_rows(ws)
    assert np.array_equal(sw, ex["scale_w"].astype(np.float32))
    assert np.array_equal(wq, ex["wq"].astype(np.int8)), wq
    acc = o.int_gemm(xq, wq)
    assert np.array_equal(acc, ex["acc"].astype(np.int32)), acc
    y = o.dequant(acc, sx, sw, b)
    assert np.array_equal(y, ex["y"]), y
    # bf16 output: the exact y rounded once to bf16 (exact rational rounding).
    yb = o.to_bf16(y)
    want = np.array([[bf16_bits_of(rn_bf16(Fraction(v))) for v in row] for row in d["expected"]["y"]],
                    np.uint16)
    assert np.array_equal(yb, want)
    # composed helpers agree with the step-by-step route
    s2, wq2, sw2 = o.prepare_weight(w, mx, d["alpha"])
    assert np.array_equal(s2, s) and np.array_equal(wq2, wq) and np.array_equal(sw2, sw)


# ---------------------------------------------------------------------------
# 2. The floor 1e-8 and degenerate rows.
# ---------------------------------------------------------------------------
def pin_floor_and_zero_rows(o):
    rng = _rng(11)
    x = _outlier_acts(rng, 5, 32)
    x[2] = 0.0                              # an all-zero token
    q, sc = o.quantize_rows(x)
    zero_scale = rn_f32(FLOOR / 127)
    assert Fraction(float(sc[2])) == zero_scale
    assert np.all(q[2] == 0)
    # the floor constant itself and the zero-row scale, bit patterns
    assert int(np.float32(float(FLOOR)).view(np.uint32)) == 0x322BCC77
    assert int(np.float32(float(zero_scale)).view(np.uint32)) == 0x2EAD26C5
    # all-zero weight column -> mw floored; all-zero weight row -> zero codes
    w = rng.standard_normal((6, 32), dtype=np.float32) * np.float32(0.02)
    w[:, 5] = 0.0
    w[3] = 0.0
    mw = o.weight_col_max(w)
    assert Fraction(float(mw[5])) == FLOOR
    mx = o.calibrate(x)
    s, wq, sw = o.prepare_weight(w, mx, 0.5)
    assert np.all(wq[3] == 0) and Fraction(float(sw[3])) == zero_scale
    # a never-seen channel (all-zero calibration column) is floored too
    xc = x.copy()
    xc[:, 7] = 0.0
    mx0 = o.calibrate(xc)
    assert mx0[7] == 0.0
    s0 = o.smoothing_factor(mx0, mw, 1.0)
    assert Fraction(float(s0[7])) == FLOOR


# ---------------------------------------------------------------------------
# 3-6. The smoothing factor: closed forms at alpha = 0, 1, 1/2, 1/4, 3/4.
# ---------------------------------------------------------------------------
def _layer(seed, m=24, n=20, k=48):
    rng = _rng(seed)
    x = _outlier_acts(rng, m, k, chans=(3, 17), mult=50.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return x, w


def pin_alpha_zero(o):
    """alpha = 0: s_j = 1 / mw_j (one binary32 division), and s, W_q and the
    weight scales do not depend on the calibration data at all."""
    x, w = _layer(21)
    mw = o.weight_col_max(w)
    s = o.smoothing_factor(o.calibrate(x), mw, 0.0)
    want = np.maximum(np.float32(1.0) / mw, np.float32(float(FLOOR)))
    assert np.array_equal(s, want)
    s1, wq1, sw1 = o.prepare_weight(w, o.calibrate(x), 0.0)
    s2, wq2, sw2 = o.prepare_weight(w, o.calibrate(x * np.float32(7.5) + np.float32(1.0)), 0.0)
    assert np.array_equal(s1, s2) and np.array_equal(wq1, wq2) and np.array_equal(sw1, sw2)


def pin_alpha_one(o):
    """alpha = 1: s_j = mx_j (independent of W), and on the calibration
    tokens every smoothed channel has max |X~_j| = 1 exactly."""
    x, w = _layer(22)
    mx = o.calibrate(x)
    s = o.smoothing_factor(mx, o.weight_col_max(w), 1.0)
    assert np.array_equal(s, mx)
    s2 = o.smoothing_factor(mx, o.weight_col_max(w * np.float32(3.0) - np.float32(0.5)), 1.0)
    assert np.array_equal(s, s2)
    xs = o.smooth_act(x, s)
    assert np.array_equal(np.abs(xs).max(axis=0), np.ones(x.shape[1], np.float32))


def pin_alpha_half(o):
    """alpha = 1/2: s_j = sqrtf(mx_j) / sqrtf(mw_j) with correctly rounded
    binary32 square roots (numpy's float32 sqrt) and one division."""
    x, w = _layer(23)
    mx = o.calibrate(x)
    mw = o.weight_col_max(w)
    s = o.smoothing_factor(mx, mw, 0.5)
    want = np.sqrt(mx.astype(np.float32)) / np.sqrt(mw.astype(np.float32))
    assert np.array_equal(s, want.astype(np.float32))


def pin_alpha_quarters(o):
    """alpha in {1/4, 3/4}: the powers are the correctly rounded binary32
    values of mx^alpha and mw^(1-alpha) (integer-root enclosures)."""
    x, w = _layer(24)
    mx = o.calibrate(x)
    mw = o.weight_col_max(w)
    for a_num in (1, 3):
        alpha = a_num / 4
        s = o.smoothing_factor(mx, mw, alpha)
        for j in range(len(mx)):
            num = rn_f32_root(Fraction(float(mx[j])), a_num, 4)
            den = rn_f32_root(Fraction(float(mw[j])), 4 - a_num, 4)
            want = max(rn_f32(num / den), FLOOR)
            assert Fraction(float(s[j])) == want, (alpha, j)


def pin_alpha_general(o):
    """alpha outside {0, 1/4, 1/2, 3/4, 1} (the page's alpha is any value in
    [0, 1], trained through a sigmoid): each power is the correctly rounded
    binary32 value of mx^alpha and mw^(1 - alpha), computed independently as
    exp(a ln x) with the standard library's decimal arithmetic at 60 digits
    (1 - alpha is exact: alpha is a binary32 number), then one binary32
    division and the floor. Values whose power lies within 2^-44 relative of
    a binary32 rounding boundary are skipped (there a binary64 pow, faithful
    to one binary64 ulp, may round either way); they are counted and must be
    rare."""
    x, w = _layer(25)
    x[:, 5] = 0.0                                   # a floored channel too
    mx = o.calibrate(x)
    mw = o.weight_col_max(w)
    checked = skipped = 0
    for alpha in (0.1, 0.3, 0.6, 0.7, 0.9, 0.05, 0.999):
        a = Fraction(float(np.float32(alpha)))
        s = o.smoothing_factor(mx, mw, float(np.float32(alpha)))
        for j in range(len(mx)):
            bx = max(Fraction(float(mx[j])), FLOOR)
            bw = Fraction(float(mw[j]))
            num = rn_f32_pow(bx, a)
            den = rn_f32_pow(bw, 1 - a)
            if num is None or den is None:
                skipped += 1
                continue
            want = max(rn_f32(num / den), FLOOR)
            assert Fraction(float(s[j])) == want, (alpha, j, float(s[j]), float(want))
            checked += 1
    assert skipped <= checked // 100, (skipped, checked)


def pin_alpha_monotone(o):
    """s_j = mx^alpha / mw^(1 - alpha) = exp(alpha (ln mx + ln mw)) / mw is
    monotone in alpha: non-decreasing where mx mw > 1, non-increasing where
    mx mw < 1. Across a sweep that mixes the closed-form exponents and the
    general ones, each step may move against that direction by at most the
    three binary32 roundings (2^-22 relative), and s passes through the
    closed-form values at alpha = 0 (1 / mw) and 1 (mx)."""
    x, w = _layer(26, k=64)
    x[:, 9] *= np.float32(1e4)                      # mx mw well above 1
    mx = o.calibrate(x)
    mw = o.weight_col_max(w)
    alphas = [0.0, 0.05, 0.1, 0.25, 0.3, 0.4, 0.5, 0.6, 0.7, 0.75, 0.8, 0.9, 1.0]
    ss = np.stack([o.smoothing_factor(mx, mw, a).astype(np.float64) for a in alphas])
    assert np.array_equal(ss[0], (np.float32(1.0) / mw).astype(np.float64))
    assert np.array_equal(ss[-1], mx.astype(np.float64))
    prod = mx.astype(np.float64) * mw.astype(np.float64)
    slack = 2.0 ** -22
    up = prod > 1.0
    assert up.any() and (~up).any()
    d = np.diff(ss, axis=0)
    assert np.all(d[:, up] >= -slack * ss[1:, up])
    assert np.all(d[:, ~up] <= slack * ss[1:, ~up])


# ---------------------------------------------------------------------------
# 7-8. Maxima: brute force and split invariance.
# ---------------------------------------------------------------------------
def pin_calibration_running_max(o):
    rng = _rng(31)
    x = _outlier_acts(rng, 40, 24, chans=(2, 9))
    x[:, 4] = -np.abs(x[:, 4])              # a channel whose max |.| is negative
    want = np.abs(x).max(axis=0)
    assert np.array_equal(o.calibrate(x), want)
    for splits in ([40], [1, 39], [13, 13, 14], [5] * 8):
        run = np.zeros(24, np.float32)
        bounds = np.cumsum([0] + splits)
        for i in reversed(range(len(splits))):      # any batch order
            o.calibrate(x[bounds[i]:bounds[i + 1]], run)
        assert np.array_equal(run, want)


def pin_weight_col_max(o):
    rng = _rng(32)
    w = rng.standard_normal((17, 21), dtype=np.float32)
    w[:, 6] = -np.abs(w[:, 6])
    want = np.maximum(np.abs(w).max(axis=0), np.float32(float(FLOOR)))
    assert np.array_equal(o.weight_col_max(w), want)


# ---------------------------------------------------------------------------
# 9. Codes and scales in exact rational arithmetic.
# ---------------------------------------------------------------------------
def _check_rows_exact(v, q, sc):
    for r in range(v.shape[0]):
        m = max(Fraction(float(abs(t))) for t in v[r])
        want_sc = rn_f32(max(m, FLOOR) / 127)
        assert Fraction(float(sc[r])) == want_sc, r
        for j in range(v.shape[1]):
            quo = rn_f32(Fraction(float(v[r, j])) / want_sc)
            c = min(127, max(-128, round_half_even(quo)))
            assert int(q[r, j]) == c, (r, j, float(v[r, j]), float(quo), int(q[r, j]), c)


def pin_codes_exact(o):
    rng = _rng(41)
    for v in (_outlier_acts(rng, 6, 40), _with_ties(rng, 6, 40),
              rng.standard_normal((5, 33), dtype=np.float32) * np.float32(1e-3)):
        q, sc = o.quantize_rows(v)
        _check_rows_exact(v, q, sc)


def pin_smoothing_exact(o):
    """X~ = RN32(X / s) and W~ = RN32(W * s), element by element."""
    x, w = _layer(42, m=6, n=5, k=20)
    mx = o.calibrate(x)
    s = o.smoothing_factor(mx, o.weight_col_max(w), 0.5)
    xs = o.smooth_act(x, s)
    ws = o.smooth_weight(w, s)
    for t in range(x.shape[0]):
        for j in range(x.shape[1]):
            assert Fraction(float(xs[t, j])) == rn_f32(Fraction(float(x[t, j])) / Fraction(float(s[j])))
    for r in range(w.shape[0]):
        for j in range(w.shape[1]):
            assert Fraction(float(ws[r, j])) == rn_f32(Fraction(float(w[r, j])) * Fraction(float(s[j])))


# ---------------------------------------------------------------------------
# 10. Invariants of the codes.
# ---------------------------------------------------------------------------
def pin_code_invariants(o):
    rng = _rng(51)
    x = _outlier_acts(rng, 30, 64, chans=(5, 40), mult=60.0)
    q, sc = o.quantize_rows(x)
    assert q.min() >= -127                         # -128 never arises
    am = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(30), am]) == 127)   # +-127 at the row max
    assert np.all(np.sign(q[np.arange(30), am]) == np.sign(x[np.arange(30), am]))
    qn, scn = o.quantize_rows(-x)                  # odd symmetry
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)
    for e in (-20, -3, 5, 30):                     # exact power-of-two scaling
        qe, sce = o.quantize_rows(x * np.float32(2.0 ** e))
        assert np.array_equal(qe, q)
        assert np.array_equal(sce, sc * np.float32(2.0 ** e))
    perm = rng.permutation(64)                     # channel permutation
    qp, scp = o.quantize_rows(x[:, perm])
    assert np.array_equal(qp, q[:, perm]) and np.array_equal(scp, sc)


# ---------------------------------------------------------------------------
# 11. The integer product.
# ---------------------------------------------------------------------------
def pin_int_gemm(o):
    rng = _rng(61)
    for m, n, k in ((1, 1, 1), (3, 5, 7), (9, 4, 33)):
        a = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
        b = rng.integers(-128, 128, size=(n, k)).astype(np.int8)
        acc = o.int_gemm(a, b)
        for t in range(m):
            for u in range(n):
                assert int(acc[t, u]) == sum(int(a[t, j]) * int(b[u, j]) for j in range(k))
        perm = rng.permutation(k)
        assert np.array_equal(o.int_gemm(a[:, perm], b[:, perm]), acc)
    # extremes: |acc| = 128^2 k with k = 4096 still fits int32
    a = np.full((2, 4096), -128, np.int8)
    acc = o.int_gemm(a, a)
    assert np.all(acc == 128 * 128 * 4096)


# ---------------------------------------------------------------------------
# 12-14. The dequantised output.
# ---------------------------------------------------------------------------
def pin_dequant_matches_simulated_forward(o):
    """The page's own formulation (dequantise both operands, multiply, add
    bias) equals acc * scale_x * scale_w + bias up to binary64 rounding."""
    rng = _rng(71)
    x = _outlier_acts(rng, 7, 96, chans=(4,))
    w = rng.standard_normal((5, 96), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(5, dtype=np.float32) * np.float32(0.01)
    s, wq, sw = o.prepare_weight(w, o.calibrate(x), 0.5)
    xq, sx, acc, y = o.linear(x, s, wq, sw, b)
    ysim = o.simulated_forward(xq, sx, wq, sw, b)
    scale = np.abs(acc.astype(np.float64) * sx[:, None] * sw[None, :]) + np.abs(b)[None, :]
    assert np.all(np.abs(y - ysim) <= 1e-12 * scale)


def pin_dequant_exact(o):
    rng = _rng(72)
    acc = rng.integers(-2 ** 30, 2 ** 30, size=(4, 3)).astype(np.int32)
    sx = (rng.random(4) * 0.1).astype(np.float32)
    sw = (rng.random(3) * 0.01).astype(np.float32)
    b = rng.standard_normal(3, dtype=np.float32)
    y = o.dequant(acc, sx, sw, b)
    for t in range(4):
        for u in range(3):
            exact = Fraction(int(acc[t, u])) * Fraction(float(sx[t])) * Fraction(float(sw[u])) + Fraction(float(b[u]))
            assert abs(Fraction(float(y[t, u])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)


def pin_bf16_rounding(o):
    rng = _rng(73)
    v = np.concatenate([rng.standard_normal(200) * 10.0 ** rng.integers(-40, 38, 200),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2.0 ** -133,
                                  3 * 2.0 ** -134, 2.0 ** -140, 0.0, -0.0, 65504.0])])
    got = o.to_bf16(v)
    for i, val in enumerate(v):
        r = rn_bf16(Fraction(float(val)))
        if r == 0:
            want = 0x8000 if np.signbit(val) else 0
        else:
            want = bf16_bits_of(r)
        assert int(got[i]) == want, (val, hex(int(got[i])), hex(want))


# ---------------------------------------------------------------------------
# 15-16. The transform is an identity; the error bound.
# ---------------------------------------------------------------------------
def pin_smoothing_identity(o):
    """(X / s)(W * s)^T = X W^T up to the binary32 rounding of X~ and W~:
    each term has relative error <= 2^-23, so per entry
    |X~ W~^T - X W^T| <= 2^-22 * sum_j |X_tj W_oj|."""
    x, w = _layer(81, m=12, n=10, k=64)
    for alpha in (0.25, 0.5, 0.75):
        s = o.smoothing_factor(o.calibrate(x), o.weight_col_max(w), alpha)
        xs = o.smooth_act(x, s).astype(np.float64)
        ws = o.smooth_weight(w, s).astype(np.float64)
        x64, w64 = x.astype(np.float64), w.astype(np.float64)
        diff = np.abs(xs @ ws.T - x64 @ w64.T)
        bound = 2.0 ** -22 * (np.abs(x64) @ np.abs(w64).T) + 1e-300
        assert np.all(diff <= bound)
        # and the smoothing really moves the outlier: max|X~| over max|X| shrinks
        assert np.abs(xs).max() < np.abs(x64).max()


def error_bound_terms(o, x, w, b, alpha):
    """Returns (err, literal_bound, provable_bound) for the docstring's
    error statement, Frobenius norms as quantization_error measures them."""
    s, wq, sw = o.prepare_weight(w, o.calibrate(x), alpha)
    xq, sx, acc, y = o.linear(x, s, wq, sw, b)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    yfp = x64 @ w64.T + b.astype(np.float64)
    err = np.linalg.norm(yfp - y)
    eps = 2.0 ** -7
    literal = eps * np.linalg.norm(w64) * np.linalg.norm(x64) + eps * np.linalg.norm(x64) * np.linalg.norm(w64)
    xs = o.smooth_act(x, s).astype(np.float64)
    ws = o.smooth_weight(w, s).astype(np.float64)
    xd = xq.astype(np.float64) * sx[:, None]
    wd = wq.astype(np.float64) * sw[:, None]
    ex = np.linalg.norm(xs - xd) / np.linalg.norm(xs)
    ew = np.linalg.norm(ws - wd) / np.linalg.norm(ws)
    resid = np.linalg.norm(xs @ ws.T - x64 @ w64.T)
    provable = (ex + ew + ex * ew) * np.linalg.norm(xs) * np.linalg.norm(ws) + resid
    return err, literal, provable


def pin_error_bound(o):
    rng = _rng(91)
    x = _outlier_acts(rng, 16, 256, chans=(3, 77, 200), mult=40.0)
    w = rng.standard_normal((128, 256), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(128, dtype=np.float32) * np.float32(0.01)
    for alpha in (0.0, 0.25, 0.5, 0.75, 1.0):
        err, literal, provable = error_bound_terms(o, x, w, b, alpha)
        assert err <= literal, (alpha, err, literal)
        assert err <= provable * (1 + 1e-9), (alpha, err, provable)


# ---------------------------------------------------------------------------
# 17. Never calibrated: s = 1, plain per-token / per-channel int8.
# ---------------------------------------------------------------------------
def pin_uncalibrated(o):
    x, w = _layer(101, m=8, n=6, k=32)
    s = o.smoothing_factor(None, o.weight_col_max(w), 0.5)
    assert np.all(s == 1.0)
    s2, wq, sw = o.prepare_weight(w, None, 0.5)
    q_plain, sc_plain = o.quantize_rows(w)
    assert np.array_equal(wq, q_plain) and np.array_equal(sw, sc_plain)
    xq, sx = o.quantize_act(x, s2)
    qx, scx = o.quantize_rows(x)
    assert np.array_equal(xq, qx) and np.array_equal(sx, scx)


# ---------------------------------------------------------------------------
# Per-tensor variant: page "quantized_linear.py", quantize_tensor (8 bits,
# range [-128, 127], one scale max|x| / 127, replaced by 1 below 1e-8) and
# QuantizedLinear (the dequantised operands multiplied, then + bias).
# ---------------------------------------------------------------------------
def _check_tensor_exact(v, q, sc):
    m = max(Fraction(float(abs(t))) for t in v.ravel())
    want = rn_f32(m / 127)
    if want < FLOOR:
        want = Fraction(1)
    assert Fraction(float(sc)) == want
    for idx, val in np.ndenumerate(v):
        quo = rn_f32(Fraction(float(val)) / want)
        c = min(127, max(-128, round_half_even(quo)))
        assert int(q[idx]) == c, (idx, float(val), int(q[idx]), c)


def pin_per_tensor_codes_exact(o):
    rng = _rng(91)
    for v in (_outlier_acts(rng, 5, 24), _with_ties(rng, 4, 16),
              rng.standard_normal((3, 7), dtype=np.float32) * np.float32(1e-3)):
        q, sc = o.quantize_tensor(v)
        _check_tensor_exact(v, q, sc)


def pin_per_tensor_replacement(o):
    """Below 1e-8 the scale is 1 (not a floored value); just above, it is
    max / 127 itself."""
    q, sc = o.quantize_tensor(np.zeros((3, 4), np.float32))
    assert sc == np.float32(1.0) and not q.any()
    v = np.array([1e-7, -5e-7, 1.2e-6], np.float32)      # 1.2e-6 / 127 < 1e-8
    q, sc = o.quantize_tensor(v)
    assert sc == np.float32(1.0) and not q.any()
    v = np.array([2e-6, -1e-6, 0.0], np.float32)          # 2e-6 / 127 > 1e-8
    q, sc = o.quantize_tensor(v)
    assert Fraction(float(sc)) == rn_f32(Fraction(float(np.float32(2e-6))) / 127)
    assert q[0] == 127 and q[2] == 0
    _check_tensor_exact(v, q, sc)


def pin_per_tensor_is_one_row(o):
    """One scale for the whole tensor: the flattened tensor quantised as a
    single row (max/127 above 1e-8, so the floor and the replacement agree);
    reshaping and permuting the tensor moves the codes with the values."""
    rng = _rng(92)
    v = _outlier_acts(rng, 6, 20, chans=(3,), mult=30.0)
    q, sc = o.quantize_tensor(v)
    qr, scr = o.quantize_rows(v.reshape(1, -1))
    assert sc == scr[0] and np.array_equal(q.reshape(1, -1), qr)
    perm = rng.permutation(v.size)
    qp, scp = o.quantize_tensor(v.ravel()[perm].reshape(10, 12))
    assert scp == sc and np.array_equal(qp.ravel(), q.ravel()[perm])
    assert np.abs(q).max() == 127 and q.min() >= -127


def pin_per_tensor_linear(o):
    """acc * sx * sw + bias equals the page's QuantizedLinear route (the
    dequantised operands multiplied, then + bias) up to binary64 rounding,
    and the integer product is the brute-force one."""
    rng = _rng(93)
    x = _outlier_acts(rng, 5, 40, chans=(2,))
    w = rng.standard_normal((6, 40), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(6, dtype=np.float32) * np.float32(0.01)
    xq, sx, wq, sw, acc, y = o.linear_per_tensor(x, w, b)
    assert np.array_equal(acc, xq.astype(np.int64) @ wq.astype(np.int64).T)
    ysim = o.simulated_forward(xq, np.full(5, sx, np.float32), wq, np.full(6, sw, np.float32), b)
    scale = np.abs(acc.astype(np.float64) * float(sx) * float(sw)) + np.abs(b)[None, :]
    assert np.all(np.abs(y - ysim) <= 1e-12 * scale)


# ---------------------------------------------------------------------------
# Weight-only int8 linear: torchao page "quantization/subclass.py",
# Int8WeightOnlyQuantizedLinearWeight (x @ int8 weights in x's type, times
# the per-output-channel scales, plus the bias).
# ---------------------------------------------------------------------------
def pin_wo_linear_exact(o):
    """Brute force in exact rational arithmetic on bf16 activations: every
    product is exact, so the binary64 sum is within 2^-50 of the exact one."""
    rng = _rng(101)
    x = _bf16_round(rng.standard_normal((3, 24), dtype=np.float32))
    wq = rng.integers(-128, 128, size=(4, 24)).astype(np.int8)
    sw = (rng.random(4, dtype=np.float32) * np.float32(0.01)).astype(np.float32)
    b = rng.standard_normal(4, dtype=np.float32)
    y = o.wo_linear(x, wq, sw, b)
    for t in range(3):
        for u in range(4):
            s = sum(Fraction(float(x[t, j])) * int(wq[u, j]) for j in range(24))
            exact = s * Fraction(float(sw[u])) + Fraction(float(b[u]))
            mag = sum(abs(Fraction(float(x[t, j])) * int(wq[u, j])) for j in range(24)) * Fraction(float(sw[u]))
            assert abs(Fraction(float(y[t, u])) - exact) <= (mag + abs(Fraction(float(b[u])))) * Fraction(1, 2 ** 50)


def pin_wo_linear_matches_integer_route(o):
    """Activations already on an int8 grid (x = xq * sx): the weight-only
    product equals the integer product scaled back, acc * sx * sw + bias."""
    rng = _rng(102)
    xq = rng.integers(-127, 128, size=(5, 40)).astype(np.int8)
    sx = np.float32(2.0 ** -7)                       # exact products and sums
    x = xq.astype(np.float32) * sx
    wq = rng.integers(-127, 128, size=(6, 40)).astype(np.int8)
    sw = (rng.random(6, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    b = rng.standard_normal(6, dtype=np.float32) * np.float32(0.1)
    y = o.wo_linear(x, wq, sw, b)
    acc = o.int_gemm(xq, wq)
    want = o.dequant(acc, np.full(5, sx, np.float32), sw, b)
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


def pin_wo_linear_structure(o):
    """Invariant under a common permutation of K; a zero weight row gives the
    bias; scaling one output channel's scale scales only that column."""
    rng = _rng(103)
    x = _bf16_round(rng.standard_normal((4, 32), dtype=np.float32))
    wq = rng.integers(-128, 128, size=(5, 32)).astype(np.int8)
    wq[2] = 0
    sw = (rng.random(5, dtype=np.float32) * np.float32(0.01) + np.float32(0.001)).astype(np.float32)
    b = rng.standard_normal(5, dtype=np.float32)
    y = o.wo_linear(x, wq, sw, b)
    perm = rng.permutation(32)
    assert np.allclose(o.wo_linear(x[:, perm], wq[:, perm], sw, b), y, rtol=1e-14, atol=1e-14)
    assert np.all(y[:, 2] == np.float64(b[2]))
    sw2 = sw.copy()
    sw2[4] *= np.float32(2.0)
    y2 = o.wo_linear(x, wq, sw2, b)
    assert np.array_equal(y2[:, :4], y[:, :4])
    assert np.allclose(y2[:, 4] - b[4], 2 * (y[:, 4] - b[4]), rtol=1e-14, atol=1e-14)


def _bf16_round(v):
    """Round float32 values to the nearest bf16 (ties to even), as float32."""
    bits = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    r = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# quantization_error (page "w8a8_smoothquant.py",
# SmoothQuantW8A8.quantization_error): the unquantised linear Y_fp and the
# measure ||Y_fp - Y_q||_F / max(||Y_fp||_F, 1e-12).
# ---------------------------------------------------------------------------
def pin_reference_linear_exact(o):
    """Dyadic inputs with few significant bits make every partial sum exact in
    binary64: the oracle must equal the exact rational x w^T + b. Random fp32
    inputs: within the binary64 summation bound of the exact value."""
    rng = _rng(131)
    m, n, k = 3, 5, 7
    x = (rng.integers(-15, 16, (m, k)) * 2.0 ** -3).astype(np.float32)
    w = (rng.integers(-31, 32, (n, k)) * 2.0 ** -6).astype(np.float32)
    b = (rng.integers(-9, 10, n) * 2.0 ** -4).astype(np.float32)
    for bias in (b, None):
        y = o.reference_linear(x, w, bias)
        for t in range(m):
            for c in range(n):
                exact = sum(Fraction(float(x[t, j])) * Fraction(float(w[c, j])) for j in range(k))
                if bias is not None:
                    exact += Fraction(float(bias[c]))
                assert Fraction(float(y[t, c])) == exact, (t, c)
    x = rng.standard_normal((4, 33), dtype=np.float32)
    w = rng.standard_normal((6, 33), dtype=np.float32)
    y = o.reference_linear(x, w, None)
    for t in range(4):
        for c in range(6):
            terms = [Fraction(float(x[t, j])) * Fraction(float(w[c, j])) for j in range(33)]
            exact = sum(terms)
            bound = 33 * 2.0 ** -53 * float(sum(abs(v) for v in terms))
            assert abs(float(Fraction(float(y[t, c])) - exact)) <= bound, (t, c)


def pin_relative_error_closed_forms(o):
    """Equal outputs give 0; y_q = y_fp (1 - 2^-e) with fp32-valued y_fp gives
    exactly 2^-e (every step scales exactly by a power of two); disjoint
    supports add in quadrature (3, 4 -> 5/3); a zero reference divides by the
    floor 1e-12."""
    rng = _rng(137)
    a = rng.standard_normal(257, dtype=np.float32).astype(np.float64)
    r, num, den = o.relative_error(a, a)
    assert r == 0.0 and num == 0.0 and den > 0
    for e in (1, 7, 20):
        d = 2.0 ** -e
        r, num, den = o.relative_error(a, a * (1.0 - d))
        assert r == d and num == d * den, (e, r)
    r, num, den = o.relative_error(np.array([3.0, 0.0]), np.array([0.0, 4.0]))
    assert (num, den) == (5.0, 3.0) and abs(r - 5.0 / 3.0) <= 2.0 ** -52
    r, num, den = o.relative_error(np.zeros(2), np.array([3.0, 4.0]))
    assert (num, den) == (5.0, 0.0) and abs(r / 5e12 - 1.0) <= 2.0 ** -52


def pin_quantization_error(o):
    """On the outlier-channel layer of the error-bound pin: the oracle's
    quantization_error times ||Y_fp||_F equals the error measured there
    independently (numpy's binary64 product), smoothing with alpha = 0.5
    beats the never-calibrated s = 1 (the method's purpose on outlier
    channels), and alpha = 0.5 stays below the provable bound."""
    rng = _rng(91)
    x = _outlier_acts(rng, 16, 256, chans=(3, 77, 200), mult=40.0)
    w = rng.standard_normal((128, 256), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(128, dtype=np.float32) * np.float32(0.01)
    mx = o.calibrate(x)
    yfp = x.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)
    q_half = o.quantization_error(x, w, b, mx, 0.5)
    err, _, provable = error_bound_terms(o, x, w, b, 0.5)
    assert abs(q_half * np.linalg.norm(yfp) - err) <= 1e-9 * err
    assert q_half * np.linalg.norm(yfp) <= provable * (1 + 1e-9)
    q_plain = o.quantization_error(x, w, b, None, 0.5)
    assert q_half < q_plain, (q_half, q_plain)




# ---------------------------------------------------------------------------
# The learnable alpha and the straight-through backward (page
# "w8a8_smoothquant.py": the docstring's V5 notes, STEQuantize /
# ste_quantize, SmoothQuantW8A8.alpha and forward).
# ---------------------------------------------------------------------------
def _ste_layer(seed, m=5, n=6, k=32, masked=False):
    """A small outlier layer, its frozen forward at alpha = sigmoid(eta) and
    an upstream gradient. With ``masked`` one channel's s_raw falls below
    the floor (never activated, huge weights), so the floor passes no
    gradient there."""
    rng = _rng(seed)
    x = _outlier_acts(rng, m, k, chans=(2, 11), mult=30.0)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.05)
    if masked:
        x[:, 7] = (rng.standard_normal(m) * 1e-6).astype(np.float32)
        w[:, 7] = (rng.standard_normal(n) * 1e12).astype(np.float32)
    b = rng.standard_normal(n, dtype=np.float32) * np.float32(0.1)
    dy = rng.standard_normal((m, n), dtype=np.float32)
    return x, w, b, dy


def _surrogate_loss(x, w, b, dy, mx, mw, eta, dx_off, dw_off):
    """sum(dy * G) for the straight-through surrogate of the quantized
    forward: G = (X / s(eta) + Dx)(W * s(eta) + Dw)^T + b, where the
    quantisation offsets Dx, Dw are held at their values at the base point
    (the estimator passes gradients through round and clamp unchanged) and
    s(eta) = max(exp(a ln mx - (1 - a) ln mw), 1e-8), a = 1/(1 + e^-eta),
    all in binary64."""
    a = 1.0 / (1.0 + np.exp(-eta))
    lmx = np.log(np.maximum(mx.astype(np.float64), float(FLOOR)))
    lmw = np.log(mw.astype(np.float64))
    s = np.maximum(np.exp(a * lmx - (1.0 - a) * lmw), float(FLOOR))
    xs = x / s[None, :] + dx_off
    ws = w * s[None, :] + dw_off
    return float(np.sum(dy * (xs @ ws.T + b[None, :])))


def pin_ste_finite_differences(o):
    """Central finite differences of the straight-through surrogate (codes
    held fixed, binary64) agree with the oracle's analytic gradients at X,
    W, the bias and eta, including a channel where the floor of s is
    active. The oracle works from binary32 alpha and s, the surrogate from
    binary64 ones, so they agree to about 1e-7; the bar is 1e-5 of each
    gradient's scale."""
    for masked, eta in ((False, 0.4), (True, -0.3), (False, 0.0)):
        x, w, b, dy = _ste_layer(140 + int(masked), masked=masked)
        mx = o.calibrate(x)
        r = o.training_step(x, w, b, mx, eta, dy)
        x64, w64, b64, dy64 = (v.astype(np.float64) for v in (x, w, b, dy))
        s64 = r["s"].astype(np.float64)
        dx_off = r["xq"].astype(np.float64) * r["sx"].astype(np.float64)[:, None] - x64 / s64[None, :]
        dw_off = r["wq"].astype(np.float64) * r["sw"].astype(np.float64)[:, None] - w64 * s64[None, :]
        mw = r["mw"]

        def L(xx=x64, ww=w64, bb=b64, ee=float(np.float32(eta))):
            return _surrogate_loss(xx, ww, bb, dy64, mx, mw, ee, dx_off, dw_off)

        # the magnitude of the surrogate's terms bounds the rounding error of
        # one evaluation (a few hundred binary64 roundings at most)
        xs = x64 / s64[None, :] + dx_off
        ws = w64 * s64[None, :] + dw_off
        mag = float(np.sum(np.abs(dy64) * (np.abs(xs) @ np.abs(ws).T + np.abs(b64)[None, :])))

        def fd(f, v, h):
            return (f(v + h) - f(v - h)) / (2 * h)

        def fd_tol(h):
            return 1e-13 * mag / h

        rng = _rng(150)
        for _ in range(12):
            t, j = rng.integers(x.shape[0]), rng.integers(x.shape[1])
            h = 1e-4 * max(1.0, abs(x64[t, j]))

            def fx(v, t=t, j=j):
                xx = x64.copy()
                xx[t, j] = v
                return L(xx=xx)
            g = fd(fx, x64[t, j], h)
            assert abs(g - r["dx"][t, j]) <= 1e-5 * np.abs(r["dx"]).max() + fd_tol(h), ("dx", t, j, g, r["dx"][t, j])
            o_, j = rng.integers(w.shape[0]), rng.integers(w.shape[1])
            h = 1e-4 * max(1e-3, abs(w64[o_, j]))

            def fw(v, o_=o_, j=j):
                ww = w64.copy()
                ww[o_, j] = v
                return L(ww=ww)
            g = fd(fw, w64[o_, j], h)
            assert abs(g - r["dw"][o_, j]) <= 1e-5 * np.abs(r["dw"]).max() + fd_tol(h), ("dw", o_, j, g, r["dw"][o_, j])
        for o_ in range(w.shape[0]):
            def fb(v, o_=o_):
                bb = b64.copy()
                bb[o_] = v
                return L(bb=bb)
            assert abs(fd(fb, b64[o_], 1e-3) - r["db"][o_]) <= 1e-9 * abs(r["db"][o_]) + fd_tol(1e-3)
        e0 = float(np.float32(eta))
        g = fd(lambda v: L(ee=v), e0, 1e-4)
        assert abs(g - r["deta"]) <= 1e-5 * abs(r["deta"]) + fd_tol(1e-4), (masked, g, r["deta"], fd_tol(1e-4))
        a = float(r["alpha"])
        assert abs(r["deta"] - r["dalpha"] * a * (1 - a)) <= 1e-15 * abs(r["dalpha"])
        if masked:
            # the floored channel: s is the floor there and ds is far from
            # zero, yet it passes nothing to alpha (the finite difference
            # above agrees)
            assert r["s"][7] == np.float32(float(FLOOR)) and abs(r["ds"][7]) > 1.0


def pin_ste_exact_quantisers_give_no_alpha_gradient(o):
    """The smoothing transform is an identity (module docstring: X~ W~^T =
    X W^T), so when both quantisers are exact (X / s and W * s already on
    their code grids) the straight-through gradient reaching s, alpha and
    eta is exactly zero, while the gradients at X and W are the plain
    linear's (dy W and dy^T X). Dyadic values make every binary64 sum
    exact."""
    rng = _rng(160)
    m, n, k = 4, 5, 16
    xq = rng.integers(-126, 127, size=(m, k)).astype(np.int8)
    wq = rng.integers(-126, 127, size=(n, k)).astype(np.int8)
    xq[np.arange(m), rng.integers(k, size=m)] = 127
    wq[np.arange(n), rng.integers(k, size=n)] = -127
    sx = (2.0 ** rng.integers(-9, -3, size=m)).astype(np.float32)
    sw = (2.0 ** rng.integers(-12, -6, size=n)).astype(np.float32)
    s = (2.0 ** rng.integers(-3, 4, size=k)).astype(np.float32)
    x = (xq.astype(np.float64) * sx[:, None] * s[None, :]).astype(np.float32)
    w = (wq.astype(np.float64) * sw[:, None] / s[None, :]).astype(np.float32)
    # the quantisers reproduce the codes exactly at this s
    q1, c1 = o.quantize_act(x, s)
    q2, c2 = o.quantize_rows(o.smooth_weight(w, s))
    assert np.array_equal(q1, xq) and np.array_equal(c1, sx) and np.array_equal(q2, wq) and np.array_equal(c2, sw)
    dy = rng.integers(-8, 9, size=(m, n)).astype(np.float32)
    mx = np.abs(x).max(axis=0)
    mw = o.weight_col_max(w)
    r = o.ste_backward(dy, x, w, s, xq, sx, wq, sw, mx, mw, np.float32(0.5))
    assert np.all(r["ds"] == 0.0) and r["dalpha"] == 0.0 and r["deta"] == 0.0
    assert np.array_equal(r["dx"], dy.astype(np.float64) @ w.astype(np.float64))
    assert np.array_equal(r["dw"], dy.astype(np.float64).T @ x.astype(np.float64))
    assert np.array_equal(r["db"], dy.astype(np.float64).sum(axis=0))


def pin_sigmoid_parametrisation(o):
    """alpha = sigmoid(eta) rounded once to binary32 (checked against a
    60-digit decimal evaluation), eta = 0 gives exactly 1/2, the page's
    initial eta round-trips alpha to within one binary32 ulp, and
    sigmoid(-eta) = 1 - sigmoid(eta) to within an ulp."""
    import decimal
    ctx = decimal.Context(prec=60)
    assert o.alpha_from_eta(0.0) == np.float32(0.5)
    assert o.eta_from_alpha(0.5) == np.float32(0.0)
    for eta in (-6.0, -2.5, -0.75, -0.1, 0.3, 1.0, 4.0, 9.0):
        e = Fraction(float(np.float32(eta)))
        ed = ctx.divide(decimal.Decimal(e.numerator), decimal.Decimal(e.denominator))
        exact = Fraction(ctx.divide(decimal.Decimal(1), ctx.add(decimal.Decimal(1), ctx.exp(-ed))))
        lo, hi = rn_f32(exact * (1 - Fraction(1, 2 ** 44))), rn_f32(exact * (1 + Fraction(1, 2 ** 44)))
        got = Fraction(float(o.alpha_from_eta(eta)))
        if lo == hi:
            assert got == lo, (eta, float(got), float(lo))
        a, a_neg = float(o.alpha_from_eta(eta)), float(o.alpha_from_eta(-eta))
        assert abs(a + a_neg - 1.0) <= 2.0 ** -23
    for alpha in (0.05, 0.25, 0.5, 0.75, 0.9):
        back = float(o.alpha_from_eta(o.eta_from_alpha(alpha)))
        assert abs(back - alpha) <= 2.0 ** -23 * max(alpha, 0.5), (alpha, back)
    # the page's guard: an initial alpha of 1 gives log(1 / 1e-6)
    assert o.eta_from_alpha(1.0) == np.float32(np.log(1e6))


def pin_aux_loss(o):
    """The docstring's auxiliary loss ||y_fp - y_q||^2 / ||y_fp||^2: zero with
    a zero gradient at y_q = y_fp; exactly 2^-2e with gradient
    -2^(1-e) y_fp / ||y_fp||^2 at y_q = y_fp (1 - 2^-e) (every step exact for
    binary32-valued y_fp in binary64, up to the final division); and its
    gradient matches central finite differences."""
    rng = _rng(170)
    y = rng.standard_normal(37, dtype=np.float32).astype(np.float64)
    loss, g = o.aux_loss_grad(y, y)
    assert loss == 0.0 and np.all(g == 0.0)
    f2 = float(np.sum(y * y))
    for e in (3, 11):
        d = 2.0 ** -e
        loss, g = o.aux_loss_grad(y, y * (1 - d))
        assert abs(loss - d * d) <= 2.0 ** -50 * d * d
        assert np.allclose(g, -2 * d * y / f2, rtol=1e-14, atol=0)
    yq = y + rng.standard_normal(37) * 0.1
    loss, g = o.aux_loss_grad(y, yq)
    for i in range(0, 37, 5):
        h = 1e-6
        p, mm = yq.copy(), yq.copy()
        p[i] += h
        mm[i] -= h
        fd = (o.aux_loss_grad(y, p)[0] - o.aux_loss_grad(y, mm)[0]) / (2 * h)
        assert abs(fd - g[i]) <= 1e-7 * np.abs(g).max()


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
