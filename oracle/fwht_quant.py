"""Online rotation + per-token INT4 of activations (oracle; test infrastructure).

Page "SpinQuant, Reproduced", Q5: R4 sits before down_proj and is applied
online as a Hadamard over the MLP width; the abstract quantizes activations to
4 bits.  Steps, in the method's order:

  1. y = x . blockdiag(H_n / sqrt(n))  (dense float64, rounded once to float32);
  2. per-token (per-row) symmetric INT4 of y (``quant.quantize_rows``);
  3. nibble packing (``quant.pack_int4``).

``had_n == 1`` means no rotation (quantization only); the rows are then the
input values converted exactly to float32.
"""

import numpy as np

from .hadamard import rotate_rows
from .quant import quantize_rows, pack_int4

__all__ = ["fwht_quant", "fwht_quant8"]


def fwht_quant(x, had_n: int):
    """Return (packed codes uint8 [M, K/2], scales float32 [M], y float32 [M, K])."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    if had_n == 1:
        y = x.astype(np.float32)
    else:
        y = rotate_rows(x, had_n).astype(np.float32)
    codes, scales = quantize_rows(y)
    return pack_int4(codes), scales, y


def fwht_quant8(x, had_n: int):
    """The 8-bit-activation variant (W4A8): the same rotation, then per-token
    symmetric INT8 (``quantize_rows`` with qmax = 127), one code per byte.
    Returns (codes int8 [M, K], scales float32 [M], y float32 [M, K])."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    y = x.astype(np.float32) if had_n == 1 else rotate_rows(x, had_n).astype(np.float32)
    codes, scales = quantize_rows(y, 127)
    return codes, scales, y
