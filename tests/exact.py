"""Exact rational arithmetic used to pin the oracle.

Rounding to a binary format is written here from its definition (nearest
representable value, ties to the even significand) on python Fractions, so
that it shares nothing with the C oracle or with numpy's float arithmetic.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

HALF = Fraction(1, 2)


def _floor_log2(a: Fraction) -> int:
    """e with 2^e <= a < 2^(e+1), a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(v: Fraction, p: int, emin: int, emax: int) -> Fraction | float:
    """Round v to nearest (ties to even) in a binary format with p significant
    bits, minimum normal exponent emin (subnormals below) and maximum
    exponent emax. Returns a Fraction, or +-inf on overflow."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), emin)
    q = Fraction(2) ** (e - (p - 1))
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def rn_f32(v) -> Fraction:
    return round_binary(Fraction(v), 24, -126, 127)


def rn_bf16(v) -> Fraction:
    return round_binary(Fraction(v), 8, -126, 127)


def round_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > HALF or (rem == HALF and fl % 2 == 1):
        fl += 1
    return fl


def f32_of(fr: Fraction) -> np.float32:
    """A Fraction that is exactly a binary32 value -> np.float32 (checked)."""
    f = np.float32(float(fr))
    assert Fraction(float(f)) == fr, "value is not a binary32 number"
    return f


def bf16_bits_of(fr: Fraction) -> int:
    """A Fraction that is exactly a bf16 value -> its 16-bit pattern."""
    f = f32_of(fr)
    b = int(np.array([f], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0
    return b >> 16


def rn_f32_root(x: Fraction, num: int, den: int, extra_bits: int = 96) -> Fraction:
    """Correctly rounded binary32 value of x^(num/den) for den in {2, 4},
    x > 0, by integer roots. Raises if the enclosure straddles a rounding
    boundary (never observed; it would need x^(num/den) within 2^-96
    relative of a binary32 midpoint)."""
    assert den in (2, 4) and x > 0
    y = x ** num
    # y = P / Q; scale so that floor(root(y * 2^(den*F))) has many bits.
    e = _floor_log2(y)
    shift = den * (extra_bits - e // den)
    scaled = y * Fraction(2) ** shift
    ip = scaled.numerator // scaled.denominator
    r = math.isqrt(ip)
    if den == 4:
        r = math.isqrt(r)
    f = shift // den
    lo = Fraction(r, 2 ** f)
    hi = Fraction(r + 1, 2 ** f)
    if lo ** den == y:
        return rn_f32(lo)
    a, b = rn_f32(lo), rn_f32(hi)
    assert a == b, "root enclosure straddles a rounding boundary"
    return a


FLOOR = rn_f32(Fraction(1, 10 ** 8))  # the floor 1e-8 as a binary32 number


def pow_enclosure(x: Fraction, a: Fraction, digits: int = 60) -> tuple[Fraction, Fraction]:
    """An interval [lo, hi] holding x^a (x > 0, a rational), from
    exp(a ln x) evaluated with the standard library's decimal module at
    ``digits`` significant digits. decimal's ln and exp are correctly
    rounded at the working precision, so a relative margin of 10^(10 -
    digits) is far wider than the evaluation's error."""
    import decimal
    ctx = decimal.Context(prec=digits)
    xd = ctx.divide(decimal.Decimal(x.numerator), decimal.Decimal(x.denominator))
    ad = ctx.divide(decimal.Decimal(a.numerator), decimal.Decimal(a.denominator))
    v = Fraction(ctx.exp(ctx.multiply(ad, ctx.ln(xd))))
    margin = Fraction(1, 10 ** (digits - 10))
    return v * (1 - margin), v * (1 + margin)


def rn_f32_pow(x: Fraction, a: Fraction, guard_bits: int = 44) -> Fraction | None:
    """The correctly rounded binary32 value of x^a, or None when x^a lies
    within 2^-guard_bits relative of a rounding boundary between two
    binary32 numbers. The guard covers a binary64 evaluation that is
    faithful (within one binary64 ulp, 2^-52) and then rounded to binary32:
    outside the guard band both routes give the same binary32 number."""
    lo, hi = pow_enclosure(x, a)
    g = Fraction(1, 2 ** guard_bits)
    r_lo, r_hi = rn_f32(lo * (1 - g)), rn_f32(hi * (1 + g))
    return r_lo if r_lo == r_hi else None
