"""Pins for the oracle's Cayley update (page "SpinQuant, Reproduced", Q5):
exact orthogonality, the closed form in two dimensions, first-order agreement
with the tangent step, and descent on a smooth loss."""

import numpy as np

import oracle
from rotation_bit_quantization_amd import synth


def _orth_err(R):
    return np.abs(R.T @ R - np.eye(R.shape[0])).max()


def test_update_stays_orthogonal_for_any_skew_direction():
    rng = np.random.default_rng(1)
    R = synth.haar_orthogonal(rng, 64).astype(np.float64)
    R = np.linalg.qr(R)[0]
    for alpha in (1e-3, 0.1, 1.0, 10.0):
        G = rng.standard_normal((64, 64))
        R2 = oracle.cayley_step(R, G, alpha)
        assert _orth_err(R2) < 1e-12
    Y = oracle.skew_descent(R, rng.standard_normal((64, 64)))
    assert np.abs(Y + Y.T).max() == 0.0


def test_two_by_two_closed_form():
    """In 2-D with R = I and Y = [[0, t], [-t, 0]], the Cayley transform is the
    rotation by 2 atan(alpha t / 2) (tan-half-angle formula)."""
    t, alpha = 0.7, 0.9
    # G chosen so that R G^T - G R^T = [[0, t], [-t, 0]] at R = I
    G = np.array([[0.0, -t / 2], [t / 2, 0.0]])
    R2 = oracle.cayley_step(np.eye(2), G, alpha)
    th = 2 * np.arctan(alpha * t / 2)
    ref = np.array([[np.cos(th), np.sin(th)], [-np.sin(th), np.cos(th)]])
    assert np.abs(R2 - ref).max() < 1e-14


def test_first_order_matches_tangent_step():
    rng = np.random.default_rng(2)
    R = np.linalg.qr(rng.standard_normal((16, 16)))[0]
    G = rng.standard_normal((16, 16))
    Y = oracle.skew_descent(R, G)
    for alpha in (1e-3, 1e-4):
        d = oracle.cayley_step(R, G, alpha) - (R + alpha * Y @ R)
        assert np.abs(d).max() < 10 * alpha ** 2 * np.abs(Y).max() ** 2


def test_descends_a_smooth_loss():
    """L(R) = ||R - T||_F^2 for a fixed orthogonal target T: gradient 2 (R - T);
    small Cayley steps decrease L monotonically and approach T."""
    rng = np.random.default_rng(3)
    T = np.linalg.qr(rng.standard_normal((8, 8)))[0]
    if np.linalg.det(T) < 0:
        T[:, 0] *= -1
    R = np.eye(8)
    losses = []
    for _ in range(200):
        losses.append(np.sum((R - T) ** 2))
        R = oracle.cayley_step(R, 2 * (R - T), 0.05)
    assert all(b <= a + 1e-12 for a, b in zip(losses, losses[1:]))
    assert losses[-1] < 1e-6 * losses[0]
    assert _orth_err(R) < 1e-12
