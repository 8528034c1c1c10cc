"""Symmetric INT4 / INT8 quantizers and nibble packing (oracle; test infrastructure).

The pages (abstract; page "SpinQuant, Reproduced" Q7/Q8) quantize weights,
activations and the KV cache to 4 bits but fix neither granularity, rounding,
clipping nor storage.  Readings taken here (one per decision):

  * symmetric absmax scale over one group: a = max |y|, s = fl32(a / 7);
  * code q = clamp(rne(fl32(y / s)), -7, 7), i.e. the float32 quotient is
    formed with IEEE division and rounded half-to-even; -8 never occurs;
  * a group whose maximum is 0 gets scale 0 and all-zero codes;
  * activation groups are whole rows (one token), weight groups are output
    channels, KV groups are one (token, head) vector of 128 values;
  * KV scales are stored as fp16: s16 = fp16_rne(fl32(a / 7)); codes use
    float32(s16) as divisor, and s16 == 0 gives all-zero codes;
  * two codes per byte, two's-complement nibbles, byte j holds code 2j in its
    low nibble and code 2j+1 in its high nibble.

The 8-bit variant (W4A8KV8, named among the evaluated settings on page
"SpinQuant, Reproduced", Q7) is read the same way with 127 in place of 7:
s = fl32(a / 127), codes clamp(rne(fl32(y / s)), -127, 127), one signed byte
per code; the KV scale is fp16_rne(fl32(a / 127)).

All decisions are taken in float32 because float32 is what decides the integer.
"""

import numpy as np

__all__ = ["quantize_rows", "quantize_given_scale", "quantize_kv_groups",
           "pack_int4", "unpack_int4"]

def quantize_given_scale(y, s, qmax: int = 7) -> np.ndarray:
    """Codes rne(fl32(y / s)) clamped to [-qmax, qmax], with s broadcast against y.

    ``y`` and ``s`` are float32.  Where s == 0 the codes are 0.
    """
    y32 = np.asarray(y, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = np.divide(y32, s32, dtype=np.float32)          # IEEE float32 division
    quot = np.where(s32 == 0, np.float32(0), quot)
    q = np.rint(quot)                                         # round half to even
    q = np.clip(q, -qmax, qmax)
    return q.astype(np.int8)


def quantize_rows(y, qmax: int = 7) -> tuple:
    """Per-row symmetric quantization: returns (codes int8 [..., K], scales float32 [...]).

    a = max_i |y_i| over the last axis, s = fl32(a / qmax) (qmax = 7 for INT4,
    127 for INT8), codes as in ``quantize_given_scale``.  ``y`` must already be
    float32 (the exact values whose quantization is being specified).
    """
    y32 = np.asarray(y, dtype=np.float32)
    a = np.max(np.abs(y32), axis=-1)
    s = np.divide(a, np.float32(qmax), dtype=np.float32)
    codes = quantize_given_scale(y32, s[..., None], qmax)
    return codes, s.astype(np.float32)


def quantize_kv_groups(y, qmax: int = 7) -> tuple:
    """Per-group quantization with an fp16 scale over the last axis.

    s16 = fp16 round-to-nearest-even of fl32(a / qmax); codes
    clamp(rne(fl32(y / float32(s16))), -qmax, qmax); s16 == 0 -> codes 0.
    Returns (codes int8, scales as float16).
    """
    y32 = np.asarray(y, dtype=np.float32)
    a = np.max(np.abs(y32), axis=-1)
    s32 = np.divide(a, np.float32(qmax), dtype=np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                          # IEEE RNE float32 -> float16
    codes = quantize_given_scale(y32, s16.astype(np.float32)[..., None], qmax)
    return codes, s16


def pack_int4(codes) -> np.ndarray:
    """Pack int8 codes in [-8, 7] along the last axis (even length) into bytes."""
    c = np.asarray(codes, dtype=np.int16)
    if c.shape[-1] % 2 != 0:
        raise ValueError("last axis must have even length to pack nibbles")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed) -> np.ndarray:
    """Inverse of ``pack_int4``: bytes [..., K/2] -> int8 codes [..., K]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out
