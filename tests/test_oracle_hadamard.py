"""Pins for oracle.hadamard (CPU only).

Each test checks the oracle against something other than itself: a library
routine (scipy's Sylvester matrix), the defining identities (H H^T = n I), a
matrix written by hand from the Paley definition (tests/golden), the textbook
butterfly FWHT, and the Kronecker identity formed with two small products.
"""

import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _textbook_fwht(v):
    """In-place iterative butterfly (a + b, a - b) at strides 1, 2, 4, ... (integer-exact)."""
    v = np.array(v, dtype=np.int64, copy=True)
    n = v.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024, 4096])
def test_sylvester_matches_scipy(n):
    assert np.array_equal(oracle.sylvester(n), scipy.linalg.hadamard(n))


@pytest.mark.parametrize("n", [2, 128, 256, 1024, 12, 24, 192, 1536])
def test_orthogonality_integer_exact(n):
    h = oracle.hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


def test_h12288_orthogonal_rows_sample():
    h = oracle.hadamard(12288)
    rows = np.random.default_rng(0).choice(12288, 24, replace=False)
    g = h[rows] @ h.T
    expect = np.zeros_like(g)
    expect[np.arange(len(rows)), rows] = 12288
    assert np.array_equal(g, expect)


def test_paley12_matches_hand_written_golden():
    lines = [ln.split() for ln in open(os.path.join(GOLDEN, "h12_paley_q11.txt"))
             if ln.strip() and not ln.startswith("#")]
    golden = np.array([[1 if c == "+" else -1 for c in ln] for ln in lines], dtype=np.int64)
    assert golden.shape == (12, 12)
    assert np.array_equal(oracle.paley12(), golden)


def test_paley12_structure_by_euler_criterion():
    """Entries re-derived with Euler's criterion x^5 = 1 (mod 11) for residues."""
    h = oracle.paley12()
    assert (h[0] == 1).all()
    assert (h[1:, 0] == -1).all()
    for a in range(11):
        for b in range(11):
            d = (b - a) % 11
            chi = 0 if d == 0 else (1 if pow(d, 5, 11) == 1 else -1)
            assert h[1 + a, 1 + b] == (1 if a == b else 0) + chi
    # skew-type: H + H^T = 2 I, and H is not symmetric (orientation matters)
    assert np.array_equal(h + h.T, 2 * np.eye(12, dtype=np.int64))
    assert not np.array_equal(h, h.T)


@pytest.mark.parametrize("n", [2, 4, 8, 32, 128, 256])
def test_dense_equals_textbook_fwht(n):
    """An FWHT equals the dense Hadamard for n <= 256 (integer inputs, exact)."""
    eye = np.eye(n, dtype=np.int64)
    assert np.array_equal(_textbook_fwht(eye), oracle.hadamard(n))
    x = np.random.default_rng(n).integers(-1000, 1000, size=(5, n))
    y = oracle.rotate_rows(x, n) * np.sqrt(n)
    assert np.allclose(y, _textbook_fwht(x), rtol=0, atol=1e-9 * np.abs(x).sum())


@pytest.mark.parametrize("k", [0, 1, 4, 10])
def test_kronecker_identity(k):
    """x . (H12 (x) H_2^k) = flatten(H12^T X H_2^k) with X = x viewed 12 x 2^k."""
    m = 1 << k
    n = 12 * m
    x = np.random.default_rng(k).integers(-50, 50, size=n)
    lhs = x @ oracle.hadamard(n)
    X = x.reshape(12, m)
    rhs = (oracle.paley12().T @ X @ scipy.linalg.hadamard(m)).reshape(-1)
    assert np.array_equal(lhs, rhs)


def test_kron_h24_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["kron_h24_ramp"]
    x = np.array(ex["x"], dtype=np.int64)
    assert list(x @ oracle.hadamard(24)) == ex["x_times_h24"]
    y = oracle.rotate_rows(x[None, :].astype(np.float64), 24)[0]
    assert np.allclose(y * np.sqrt(24), ex["x_times_h24"], rtol=0, atol=1e-11)


def test_rotation_is_norm_preserving_and_blockwise():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 12288 * 2))
    y = oracle.rotate_rows(x, 12288)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # block-diagonal along the row: each half rotates independently
    y0 = oracle.rotate_rows(x[:, :12288], 12288)
    assert np.allclose(y[:, :12288], y0, rtol=0, atol=1e-12)


def test_supported_orders():
    ok = [1, 2, 4, 128, 256, 16384, 12, 24, 12288]
    bad = [0, 3, 6, 36, 32768, 24576, 12 * 2048, 100]
    assert all(oracle.supported_had_n(n) for n in ok)
    assert not any(oracle.supported_had_n(n) for n in bad)
