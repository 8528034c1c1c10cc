"""KV-path rotation + INT4 KV cache (oracle; test infrastructure).

Page "SpinQuant, Reproduced", Q5: R3 sits in the KV path between operations
that do not commute, so it is an online Hadamard; the abstract quantizes the
KV cache to 4 bits.  Readings:

  * R3 acts head-wise: every (token, head) vector of D = 128 values is rotated
    by H_128 / sqrt(128) as a row vector; Q and K both receive it, which
    leaves Q K^T unchanged in full precision; V is not rotated online
    (R2 is folded into the value weights);
  * the rotated (or, for V, unrotated) vector is one quantization group with an
    fp16 scale (``quant.quantize_kv_groups``); Q is rotated but not quantized.
"""

import numpy as np

from .hadamard import rotate_rows
from .quant import quantize_kv_groups, pack_int4

__all__ = ["kv_quant", "kv_quant8"]


def kv_quant(x, rotate: bool, quantize: bool = True):
    """x [T, H, D] -> (codes uint8 [T, H, D/2] | None, scales fp16 [T, H] | None, y fp32).

    ``y`` is the float32 vector that was (or would be) quantized: the rotated
    values rounded once to float32 when ``rotate``, the exact input otherwise.
    """
    x = np.asarray(x)
    if x.ndim != 3:
        raise ValueError("x must be [T, H, D]")
    D = x.shape[-1]
    if rotate:
        y = rotate_rows(x, D).astype(np.float32)
    else:
        y = x.astype(np.float32)
    if not quantize:
        return None, None, y
    codes, s16 = quantize_kv_groups(y)
    return pack_int4(codes), s16, y


def kv_quant8(x, rotate: bool, quantize: bool = True):
    """The 8-bit KV variant (KV8): the same head-wise rotation, then per
    (token, head) INT8 with an fp16 scale (``quantize_kv_groups`` with
    qmax = 127).  Returns (codes int8 [T, H, D] | None, scales fp16 | None, y fp32)."""
    x = np.asarray(x)
    if x.ndim != 3:
        raise ValueError("x must be [T, H, D]")
    y = rotate_rows(x, x.shape[-1]).astype(np.float32) if rotate else x.astype(np.float32)
    if not quantize:
        return None, None, y
    codes, s16 = quantize_kv_groups(y, 127)
    return codes, s16, y
