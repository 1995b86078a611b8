"""Exact rational arithmetic with explicit binary32 rounding (test-side only).

Used to pin the oracle against something other than NumPy's float32: every
fp32 operation is evaluated exactly with ``fractions.Fraction`` and then rounded
to the nearest binary32 value (ties to even, subnormals included).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

_EMIN = -126          # smallest normal exponent of binary32
_P = 24               # significand bits of binary32
_MAXF = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127


def f32_round(v: Fraction) -> Fraction:
    """Round an exact rational to binary32 (RNE). Overflow raises."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, _EMIN)
    ulp = Fraction(2) ** (e - (_P - 1))
    m = round(a / ulp)          # Fraction.__round__ rounds half to even
    r = m * ulp
    if r > _MAXF:
        raise OverflowError("binary32 overflow")
    return sign * r


def frac(x) -> Fraction:
    return Fraction(float(x))


def rne_int(v: Fraction) -> int:
    return int(round(v))


def quant_row_exact(row_f32):
    """Per-row symmetric INT8 quant, exactly: s = fl32(amax/127), q = RNE(fl32(x/s))."""
    xs = [frac(v) for v in row_f32]
    amax = max(abs(v) for v in xs)
    s = f32_round(amax / 127)
    if s == 0:
        return s, [0] * len(xs)
    q = [max(-127, min(127, rne_int(f32_round(v / s)))) for v in xs]
    return s, q


def to_f32(v: Fraction) -> np.float32:
    return np.float32(float(v))
