"""Exact rational arithmetic with explicit IEEE-754 rounding, for pinning the oracle.

These helpers take decisions the slow, independent way: a real value is held
as a ``fractions.Fraction`` and rounded to the binary32 / binary16 grid by
locating its exponent and rounding the scaled significand half-to-even.  They
share nothing with numpy's float32 arithmetic, so agreement with the oracle's
float32 decisions is evidence, not a tautology.
"""

from fractions import Fraction
import math

import numpy as np


def _round_half_even(v: Fraction) -> int:
    n = math.floor(v)
    rem = v - n
    if rem > Fraction(1, 2):
        return n + 1
    if rem < Fraction(1, 2):
        return n
    return n if n % 2 == 0 else n + 1


def round_to_binary(v: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round v to the nearest value of a binary format with ``mant_bits`` explicit
    significand bits and normal exponents [emin, emax], ties to even.
    Overflow returns +-inf as a float."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix up log2 rounding so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                                   # subnormal grid below emin
    ulp = Fraction(2) ** (e - mant_bits)
    n = _round_half_even(a / ulp)
    r = n * ulp
    if r >= Fraction(2) ** (emax + 1):
        return Fraction(sign) * Fraction(10) ** 400      # marker for overflow
    return sign * r


def to_f32(v: Fraction) -> Fraction:
    return round_to_binary(v, 23, -126, 127)


def to_f16(v: Fraction) -> Fraction:
    return round_to_binary(v, 10, -14, 15)


def frac(x) -> Fraction:
    """Exact Fraction of a numpy / Python float (any binary format)."""
    return Fraction(float(x))


def quantize_exact(y_f32_values, scale: Fraction):
    """rne(fl32(y / s)) clamped to [-7, 7] for each value, exact route; s == 0 -> 0."""
    out = []
    for y in y_f32_values:
        if scale == 0:
            out.append(0)
            continue
        quot = to_f32(frac(y) / scale)
        q = _round_half_even(quot)
        out.append(max(-7, min(7, q)))
    return out


def scale_exact(y_f32_values) -> Fraction:
    """fl32(max|y| / 7), exact route."""
    a = max(abs(frac(y)) for y in y_f32_values)
    return to_f32(a / 7)


def f32(v: Fraction) -> np.float32:
    return np.float32(float(v))
