"""Pins for the 8-bit variant of the oracle (W4A8KV8, page "SpinQuant,
Reproduced", Q7 names it among the evaluated settings): the quantizer with
qmax = 127 against an exact rational route, a worked example, invariants, the
KV fp16 scale rule, and the W4A8 product by brute force."""

from fractions import Fraction

import numpy as np

import oracle
from tests import exact


def _quantize8_exact(values, scale):
    out = []
    for y in values:
        if scale == 0:
            out.append(0)
            continue
        q = exact._round_half_even(exact.to_f32(exact.frac(y) / scale))
        out.append(max(-127, min(127, q)))
    return out


def test_worked_example_h4():
    """x = [1, 2, 3, 4] through H_4 / 2 -> y = [5, -1, -2, 0]; s = fl32(5 / 127);
    y / s = [127, -25.4, -50.8, 0] -> q = [127, -25, -51, 0]."""
    codes, s, y = oracle.fwht_quant8(np.array([[1, 2, 3, 4]], np.float32), 4)
    assert y.tolist() == [[5.0, -1.0, -2.0, 0.0]]
    assert Fraction(float(s[0])) == exact.to_f32(Fraction(5, 127))
    assert codes.tolist() == [[127, -25, -51, 0]]
    assert codes.dtype == np.int8


def test_quantizer_matches_exact_route():
    rng = np.random.default_rng(11)
    y = (rng.standard_normal((24, 40)) * np.exp(rng.uniform(-8, 8, (24, 1)))).astype(np.float32)
    y[3, :] = 0.0                                  # zero row -> scale 0, codes 0
    y[5, 7] = -y[5].max() * 3                      # negative absmax
    codes, s = oracle.quantize_rows(y, 127)
    for r in range(y.shape[0]):
        se = exact.to_f32(max(abs(exact.frac(v)) for v in y[r]) / 127)
        assert Fraction(float(s[r])) == se
        assert codes[r].tolist() == _quantize8_exact(y[r], se)


def test_quantizer_invariants():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((16, 64)).astype(np.float32)
    q, s = oracle.quantize_rows(y, 127)
    qn, _ = oracle.quantize_rows(-y, 127)
    q2, s2 = oracle.quantize_rows(y * np.float32(8.0), 127)
    assert np.array_equal(qn, -q)                                      # odd symmetry
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(8.0))   # power-of-2 scale
    assert (np.abs(q).max(axis=1) == 127).all()                        # absmax maps to 127
    am = np.argmax(np.abs(y), axis=1)
    assert (np.abs(q[np.arange(16), am]) == 127).all()
    err = np.abs(y - q.astype(np.float64) * s[:, None])
    assert (err <= s[:, None] * (0.5 + 1e-5)).all()                    # round-to-nearest bound


def test_kv8_scale_rule():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((6, 3, 128)) * 4).astype(np.float16)
    codes, s16, y = oracle.kv_quant8(x, rotate=True)
    for t in range(6):
        for h in range(3):
            a = max(abs(exact.frac(v)) for v in y[t, h])
            se = exact.to_f16(exact.to_f32(a / 127))
            assert Fraction(float(s16[t, h])) == se
            assert codes[t, h].tolist() == _quantize8_exact(y[t, h], se)


def test_w4a8_gemm_brute_force():
    rng = np.random.default_rng(14)
    qx = rng.integers(-127, 128, size=(5, 96)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(3, 96)).astype(np.int8)
    sx = rng.random(5).astype(np.float32)
    sw = rng.random(3).astype(np.float32)
    y, acc = oracle.w4a8_gemm(qx, sx, oracle.pack_int4(qw), sw)
    for m in range(5):
        for n in range(3):
            a = sum(int(qx[m, k]) * int(qw[n, k]) for k in range(96))
            assert acc[m, n] == a
            assert y[m, n] == np.float32(np.float32(np.float32(a) * sx[m]) * sw[n])
