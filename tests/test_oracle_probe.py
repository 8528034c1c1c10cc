"""Pins for the rotation-choice probe's reading of "randomised Hadamard"
(page "SpinQuant, Reproduced", Q3), on the oracle, CPU only.

With symmetric absmax quantizers per token and per output channel, random
signs applied after the Hadamard (R = H D) pass through the codes and cancel in
the product: the W4A4 output equals the plain Hadamard's bit for bit.  Signs
applied to the input channels before it (R = D H) change the quantized
operands and therefore the error.  The probe uses the latter."""

import numpy as np

import oracle
from rotation_bit_quantization_amd import synth


def _layer_output(x, w, R):
    K = x.shape[1]
    _, xq, xs = oracle.fold_rotation(np.ascontiguousarray(x.T), R, K)   # per-token codes of x R
    _, wq, ws = oracle.fold_rotation(w, R, K)
    y, acc = oracle.w4a4_gemm(xq, xs, wq, ws)
    return y, acc, xq, wq


def test_signs_after_hadamard_cancel_exactly():
    cfg = synth.probe_config(T=48, K=128, N=64, draws=2)
    x, w = cfg["x"], cfg["w"]
    H = (oracle.hadamard(128) / np.sqrt(128.0)).astype(np.float32)
    y0, acc0, xq0, wq0 = _layer_output(x, w, H)
    for s in cfg["signs"]:
        y1, acc1, xq1, wq1 = _layer_output(x, w, (H * s[None, :]).astype(np.float32))   # H diag(s)
        assert np.array_equal(acc0, acc1) and np.array_equal(y0, y1)
        # the codes themselves differ exactly by the signs
        c0, c1 = oracle.unpack_int4(xq0), oracle.unpack_int4(xq1)
        assert np.array_equal(c1, c0 * s[None, :].astype(np.int64))


def test_signs_before_hadamard_change_the_codes():
    cfg = synth.probe_config(T=48, K=128, N=64, draws=2)
    x, w = cfg["x"], cfg["w"]
    H = (oracle.hadamard(128) / np.sqrt(128.0)).astype(np.float32)
    _, acc0, _, _ = _layer_output(x, w, H)
    s = cfg["signs"][0]
    _, acc1, _, _ = _layer_output(x, w, (s[:, None] * H).astype(np.float32))            # diag(s) H
    assert not np.array_equal(acc0, acc1)


def test_rotation_leaves_the_full_precision_product_unchanged():
    """The invariance the probe relies on (page "SpinQuant, Reproduced", Q1):
    (x R)(R^T w) = x w for the rotations it draws, within float32 rounding."""
    cfg = synth.probe_config(T=48, K=128, N=64, draws=2)
    x, w = cfg["x"].astype(np.float64), cfg["w"].astype(np.float64)
    H = oracle.hadamard(128) / np.sqrt(128.0)
    for R in (cfg["haar"][0].astype(np.float64), cfg["signs"][0][:, None] * H):
        got = (x @ R) @ (R.T @ w)
        ref = x @ w
        assert np.linalg.norm(got - ref) <= 1e-4 * np.linalg.norm(ref)
