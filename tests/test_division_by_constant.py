"""The kernels divide a group's absmax by 7 (or 127) without a division
sequence: q = fl32(a * rd) with rd = fl32(1 / d), r = fma(-q, d, a), then
fma(r, rd, q).  The scale is part of the bit-exact contract, so this checks
that the three roundings give the IEEE quotient fl32(a / d) for every float32
significand (a in [1, 2); each step scales exactly with a power of two while
the quotient stays normal).

float32 rounding is emulated in float64, where every intermediate here is
exact except possibly the last sum (up to 54 bits for d = 127); wherever that
sum or the float64 reference quotient lies within 2^-50 of a float32 midpoint
the rounding is redone with exact rationals.
"""
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

HEADER = os.path.join(os.path.dirname(__file__), "..", "rotation_bit_quantization_amd", "csrc",
                      "spin_device.h")


def _round_f32_exact(x):
    """Round a positive Fraction to the nearest float32 (ties to even)."""
    e = math.floor(math.log2(x))
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    scale = Fraction(2) ** (23 - e)
    n = x * scale
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return Fraction(fl) / scale


def _near_midpoint(v64):
    """float64 values within 2^-50 (relative) of a float32 rounding midpoint."""
    r = v64.astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    r64 = r.astype(np.float64)
    mid = np.where(v64 >= r64, (r64 + up) / 2, (r64 + dn) / 2)
    return np.abs(v64 - mid) <= np.abs(v64) * 2.0 ** -50


@pytest.mark.parametrize("d", [7, 127])
def test_three_roundings_give_the_ieee_quotient(d):
    rd = np.float32(1.0) / np.float32(d)
    M = np.arange(1 << 23, 1 << 24, dtype=np.int64)
    a = M.astype(np.float64) * 2.0 ** -23                       # every significand, exact
    q = (a * np.float64(rd)).astype(np.float32)                 # 48-bit product: exact, one rounding
    r64 = a - np.float64(d) * q.astype(np.float64)              # exact in float64
    r = r64.astype(np.float32)
    assert np.array_equal(r.astype(np.float64), r64)            # the FMA's result is exact
    s64 = r.astype(np.float64) * np.float64(rd) + q.astype(np.float64)
    got = s64.astype(np.float32)
    ref64 = a / d
    ref = ref64.astype(np.float32)
    for i in np.nonzero(_near_midpoint(s64))[0]:
        ex = Fraction(float(r[i])) * Fraction(float(rd)) + Fraction(float(q[i]))
        got[i] = np.float32(float(_round_f32_exact(ex)))
    for i in np.nonzero(_near_midpoint(ref64))[0]:
        ref[i] = np.float32(float(_round_f32_exact(Fraction(int(M[i]), (1 << 23) * d))))
    # the float64 shortcut for the reference, spot-checked with exact rationals
    for i in np.random.default_rng(d).integers(0, len(M), 300):
        assert Fraction(float(ref[i])) == _round_f32_exact(Fraction(int(M[i]), (1 << 23) * d))
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, f"d={d}: {len(bad)} significands differ, first a={a[bad[:3]]}"


def test_header_constants_are_the_rounded_reciprocals():
    text = open(HEADER).read()
    for name, d in (("kRcpSeven", 7), ("kRcpQmax8", 127)):
        m = re.search(r"constexpr float %s = ([0-9a-fx.p+-]+)f;" % name, text)
        assert m, name
        assert float.fromhex(m.group(1)) == float(np.float32(1.0) / np.float32(d))


def test_a_single_rounding_of_the_sum_can_differ():
    """Why the kernels keep the float32 quotient before converting to fp16: rounding
    q + r * rd straight to fp16 (as a fused fma-to-fp16 would) differs from
    fp16(fl32(a / 7)) for some a, e.g. where fl32(a / 7) sits on an fp16 tie."""
    rd = np.float32(1.0) / np.float32(7)
    M = np.arange(1 << 23, 1 << 24, dtype=np.int64)
    a = M.astype(np.float64) * 2.0 ** -23
    q = (a * np.float64(rd)).astype(np.float32)
    r = (a - 7.0 * q.astype(np.float64)).astype(np.float32)
    s64 = r.astype(np.float64) * np.float64(rd) + q.astype(np.float64)
    twice = s64.astype(np.float32).astype(np.float16)
    once = s64.astype(np.float16)           # float64 -> fp16 directly: one rounding of the sum
    assert (twice != once).any()
