"""Pins for oracle.quant / oracle.fwht_quant (CPU only).

The quantizer is checked against an exact-rational route (tests/exact.py) that
rounds with its own IEEE rule, against hand-worked examples, and against the
invariants a symmetric absmax quantizer must satisfy.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _examples():
    return json.load(open(os.path.join(GOLDEN, "worked_examples.json")))


def test_worked_example_rotate_quant_pack():
    ex = _examples()["rotate_quant_h4"]
    x = np.array([ex["x"]], dtype=np.float32)
    packed, scales, y = oracle.fwht_quant(x, 4)
    assert y[0].tolist() == ex["y"]
    assert hex(scales.view(np.uint32)[0]) == ex["scale_f32_hex"]
    assert oracle.unpack_int4(packed)[0].tolist() == ex["codes"]
    assert packed[0].tolist() == ex["packed"]


def test_rne_ties():
    ex = _examples()["rne_ties"]
    t = np.array(ex["t"], dtype=np.float32)
    # with s = 1 the quotient is t itself
    assert oracle.quantize_given_scale(t, np.float32(1.0)).tolist() == ex["q"]


def test_quantizer_matches_exact_rational_route():
    rng = np.random.default_rng(3)
    for trial in range(40):
        n = int(rng.integers(2, 40))
        y = (rng.standard_normal(n) * 10.0 ** rng.integers(-3, 4)).astype(np.float32)
        if trial % 5 == 0:
            y[rng.integers(n)] *= 50                       # outlier
        codes, s = oracle.quantize_rows(y[None, :])
        s_ex = exact.scale_exact(y)
        assert Fraction(float(s[0])) == s_ex
        assert codes[0].tolist() == exact.quantize_exact(y, s_ex)


def test_quantizer_near_ties_exact_route():
    """Values placed at float32 neighbours of (k + 1/2) * s: the decision must be
    the one the specification (fl32 quotient, then round-half-even) gives."""
    rng = np.random.default_rng(11)
    checked = 0
    for a in [1.0, 3.0, 0.7, 123.456, 5e-3]:
        a32 = np.float32(a)
        s = np.float32(a32 / np.float32(7))
        s_ex = Fraction(float(s))
        vals = [a32]
        for k in range(-7, 7):
            centre = np.float32((k + 0.5) * float(s))
            for d in range(-3, 4):
                v = centre
                for _ in range(abs(d)):
                    v = np.nextafter(v, np.float32(np.inf if d > 0 else -np.inf))
                if abs(v) <= a32:
                    vals.append(np.float32(v))
        y = np.array(vals, dtype=np.float32)
        rng.shuffle(y)
        codes, s_o = oracle.quantize_rows(y[None, :])
        assert Fraction(float(s_o[0])) == s_ex
        assert codes[0].tolist() == exact.quantize_exact(y, s_ex)
        checked += y.size
    assert checked > 300


def test_quantizer_invariants():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((16, 96)) * 3).astype(np.float32)
    y[:, 7] *= 40
    codes, s = oracle.quantize_rows(y)
    # symmetric
    c_neg, s_neg = oracle.quantize_rows(-y)
    assert np.array_equal(c_neg, -codes) and np.array_equal(s_neg, s)
    # invariant to power-of-two rescaling
    for j in (-5, 3):
        c2, s2 = oracle.quantize_rows(y * np.float32(2.0 ** j))
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))
    # the absmax element maps to +-7, codes stay within [-7, 7]
    am = np.argmax(np.abs(y), axis=1)
    assert (np.abs(codes[np.arange(16), am]) == 7).all()
    assert codes.min() >= -7 and codes.max() <= 7
    # reconstruction error at most half a step (plus float32 slack)
    err = np.abs(y - codes.astype(np.float32) * s[:, None])
    assert (err <= s[:, None] * 0.5 * (1 + 1e-6) + 1e-30).all()


def test_zero_row_and_pack_roundtrip():
    y = np.zeros((2, 8), dtype=np.float32)
    y[1, 3] = -2.0
    codes, s = oracle.quantize_rows(y)
    assert s[0] == 0 and (codes[0] == 0).all()
    assert codes[1, 3] == -7
    c = np.random.default_rng(0).integers(-8, 8, size=(5, 64)).astype(np.int8)
    p = oracle.pack_int4(c)
    assert p.shape == (5, 32)
    assert np.array_equal(oracle.unpack_int4(p), c)
    # byte layout: low nibble = even code, high nibble = odd code
    assert oracle.pack_int4(np.array([[1, -2]], np.int8))[0, 0] == (1 | (0xE << 4))


def test_kv_fp16_scale_rule_exact_route():
    """s16 = fp16_rne(fl32(a/7)); codes divide by float(s16)."""
    rng = np.random.default_rng(9)
    for _ in range(50):
        y = (rng.standard_normal(128) * 10.0 ** rng.integers(-2, 3)).astype(np.float32)
        codes, s16 = oracle.quantize_kv_groups(y[None, :])
        s_ex = exact.to_f16(exact.scale_exact(y))
        assert Fraction(float(s16[0])) == s_ex
        assert codes[0].tolist() == exact.quantize_exact(y, s_ex)


def test_kv_scale_underflow_edges():
    # a/7 between the smallest fp16 subnormals: s16 rounds far below a/7 and the clamp acts
    a = np.float32(1.4 * 2.0 ** -24 * 7)
    y = np.array([[a, -a / 2, a / 7, 0]], dtype=np.float32)
    codes, s16 = oracle.quantize_kv_groups(y)
    assert float(s16[0]) == 2.0 ** -24
    assert codes[0].tolist() == exact.quantize_exact(y[0], Fraction(2) ** -24)
    assert codes[0, 0] == 7                               # 9.8 clamped
    # a/7 below half the smallest subnormal: s16 == 0 -> all codes 0
    y0 = np.array([[np.float32(2.0 ** -27), np.float32(-2.0 ** -28)]], dtype=np.float32)
    c0, s0 = oracle.quantize_kv_groups(y0)
    assert float(s0[0]) == 0.0 and (c0 == 0).all()


@pytest.mark.parametrize("had_n", [1, 2, 32, 256, 12, 96])
def test_fwht_quant_composition(had_n):
    """fwht_quant = dense rotation rounded once to fp32, then the row quantizer."""
    rng = np.random.default_rng(had_n)
    x = rng.standard_normal((4, 768)).astype(np.float16)
    packed, s, y = oracle.fwht_quant(x, had_n)
    y_ref = oracle.rotate_rows(x, had_n).astype(np.float32) if had_n > 1 else x.astype(np.float32)
    assert np.array_equal(y, y_ref)
    codes, s_ref = oracle.quantize_rows(y_ref)
    assert np.array_equal(oracle.unpack_int4(packed), codes) and np.array_equal(s, s_ref)
