"""Offline fold of a rotation into a weight + per-channel INT4 (oracle; test infra).

Page "SpinQuant, Reproduced", Q1 and Q5: a pre-norm transformer is invariant
to an orthogonal change of basis of its hidden state, so R1 (residual) and R2
(head-wise, value path) are merged into the adjacent weights and cost nothing
at runtime; R4's inverse is merged into down_proj.  With activations rotated as
row vectors, x -> x R, the matching weight is W' = R^T W, so that
(x R)(R^T W) = x W.

Readings:
  * W is stored [K][N] (input features x output features);
  * the rotation is block-diagonal, B = blockdiag(R, ..., R) with square blocks
    of size r dividing K (r = K for R1, r = 128 for R2); ``R is None`` selects
    the library Hadamard H_r / sqrt(r) (used for R4 on down_proj);
  * W' = B^T W is formed in float64 and rounded once to float32;
  * weights are quantized per output channel (column n of W') with the same
    absmax / 7, round-half-even, clamp +-7 rule as activations, and stored
    output-channel-major, [N][K/2] packed bytes plus [N] float32 scales.
"""

import numpy as np

from .hadamard import hadamard
from .quant import quantize_rows, pack_int4

__all__ = ["block_rotation", "fold_rotation"]


def block_rotation(R, r_block: int) -> np.ndarray:
    """The float64 r x r block used by the fold: R itself, or H_r / sqrt(r) if R is None."""
    if R is None:
        return hadamard(r_block).astype(np.float64) / np.sqrt(np.float64(r_block))
    R64 = np.asarray(R, dtype=np.float64)
    if R64.shape != (r_block, r_block):
        raise ValueError("R must be r_block x r_block")
    return R64


def fold_rotation(W, R, r_block: int):
    """Return (W_rot float32 [K, N], Wq uint8 [N, K/2], w_scale float32 [N])."""
    W64 = np.asarray(W, dtype=np.float64)
    K, N = W64.shape
    if K % r_block != 0:
        raise ValueError("K must be a multiple of r_block")
    B = block_rotation(R, r_block)
    out = np.empty_like(W64)
    for b0 in range(0, K, r_block):
        out[b0:b0 + r_block] = B.T @ W64[b0:b0 + r_block]
    w_rot = out.astype(np.float32)
    codes, scales = quantize_rows(w_rot.T)          # one group per output channel
    return w_rot, pack_int4(codes), scales
