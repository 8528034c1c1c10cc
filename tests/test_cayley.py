"""R2 learning with Cayley SGD (rotation_bit_quantization_amd.cayley), CPU:
the update equals the oracle's, the straight-through objective equals the
oracle's W4A4 layer error in its forward value, and a short run lowers the
objective while the rotation stays orthogonal to float64 rounding."""

import numpy as np
import torch

import oracle
from rotation_bit_quantization_amd import cayley, synth


def test_update_matches_oracle():
    rng = np.random.default_rng(5)
    R = np.linalg.qr(rng.standard_normal((32, 32)))[0]
    G = rng.standard_normal((32, 32))
    for alpha in (1e-3, 0.3, 2.0):
        got = cayley.cayley_update(torch.as_tensor(R), torch.as_tensor(G), alpha).numpy()
        assert np.abs(got - oracle.cayley_step(R, G, alpha)).max() < 1e-12


def test_ste_objective_forward_is_the_w4a4_layer_error():
    """Forward value of the training objective = squared relative error of the
    oracle's W4A4 pipeline (fold of x^T and of w with blockdiag(R2), int64 GEMM,
    float32 epilogue), up to float32-vs-float64 rounding of the operands."""
    cfg = synth.r2_config(T=64, heads=4, head_dim=32, N=48, draws=1)
    x, w, heads, d = cfg["x"], cfg["w"], cfg["heads"], cfg["head_dim"]
    R = (cfg["signs"][0][:, None] * oracle.hadamard(d) / np.sqrt(d)).astype(np.float32)
    loss = cayley.ste_layer_loss(torch.as_tensor(x.astype(np.float64)), torch.as_tensor(w.astype(np.float64)),
                                 torch.as_tensor(R.astype(np.float64)), heads).item()
    _, xq, xs = oracle.fold_rotation(np.ascontiguousarray(x.T), R, d)
    _, wq, ws = oracle.fold_rotation(w, R, d)
    y, _ = oracle.w4a4_gemm(xq, xs, wq, ws)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert abs(loss ** 0.5 - err) <= 2e-3 * err


def test_short_run_descends_and_stays_orthogonal():
    cfg = synth.r2_config(T=128, heads=8, head_dim=64, N=64, draws=1)
    d = cfg["head_dim"]
    R0 = cfg["signs"][0][:, None] * oracle.hadamard(d) / np.sqrt(d)
    R, hist = cayley.learn_r2(cfg["x"], cfg["w"], R0, cfg["heads"], iters=25, lr=0.2)
    assert min(hist[5:]) < hist[0]
    assert np.abs(R.T @ R - np.eye(d)).max() < 1e-12
