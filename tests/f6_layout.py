"""Host encoder and decoder of the FP6 operand layout of activation codes,
written from its definition in include/libspin.h (code q of row r, column k:
field u = q + 8 in region (r / 32) * (K / 64) + k / 64, at byte
((k % 64) / 32) * 768 + (r % 32) * 24 + ((k % 32) / 16) * 12, field
sigma(k % 16) of those 12 bytes, field p at bits 6p .. 6p + 5 of the 96-bit
little-endian number).  Test infrastructure only."""

import numpy as np

SIGMA = np.array([0, 1, 12, 2, 3, 14, 4, 5, 11, 6, 7, 13, 8, 9, 15, 10])


def nbytes(M, K):
    return ((M + 31) // 32) * (K // 64) * 1536


def _fields_of_96(words):
    """words [..., 3] uint32 (little-endian 96-bit numbers) -> fields [..., 16] (6 bits each)."""
    lo = words[..., 0].astype(np.uint64) | (words[..., 1].astype(np.uint64) << np.uint64(32))
    hi = words[..., 2].astype(np.uint64)
    out = np.empty(words.shape[:-1] + (16,), np.int64)
    for p in range(16):
        b = 6 * p
        if b + 6 <= 64:
            f = (lo >> np.uint64(b)) & np.uint64(63)
        elif b >= 64:
            f = (hi >> np.uint64(b - 64)) & np.uint64(63)
        else:                                   # straddles bit 64
            f = ((lo >> np.uint64(b)) | (hi << np.uint64(64 - b))) & np.uint64(63)
        out[..., p] = f.astype(np.int64)
    return out


def decode(buf, M, K):
    """Bytes of the layout -> codes int8 [M, K]; also checks that every field
    of rows 0 .. M - 1 has its top two bits zero (the rows that pad the last
    block of 32 are not part of the contract: nothing writes them)."""
    RB, KS = (M + 31) // 32, K // 64
    b = np.asarray(buf, np.uint8).reshape(RB, KS, 2, 32, 2, 12)
    words = b.reshape(RB, KS, 2, 32, 2, 3, 4).view("<u4").reshape(RB, KS, 2, 32, 2, 3)
    fields = _fields_of_96(words)                       # [RB, KS, half, row, g, p]
    real = (np.arange(RB)[:, None] * 32 + np.arange(32)[None, :]) < M       # [RB, row]
    assert (fields >> 4 == 0)[real[:, None, None, :, None, None].repeat(KS, 1).repeat(2, 2)
                               .repeat(2, 4).repeat(16, 5)].all(), "a field's top bits are set"
    codes_by_j = fields[..., SIGMA] - 8                 # [RB, KS, half, row, g, j]
    c = codes_by_j.transpose(0, 3, 1, 2, 4, 5).reshape(RB * 32, K)   # row, then k = ks*64+half*32+g*16+j
    return c[:M].astype(np.int8)


def encode(codes):
    """codes int [M, K] in [-8, 7] -> bytes of the layout (rows past M zero codes)."""
    codes = np.asarray(codes, np.int64)
    M, K = codes.shape
    RB, KS = (M + 31) // 32, K // 64
    c = np.zeros((RB * 32, K), np.int64)
    c[:M] = codes
    u = (c + 8).reshape(RB, 32, KS, 2, 2, 16).transpose(0, 2, 3, 1, 4, 5)   # [RB, KS, half, row, g, j]
    fields = np.empty_like(u)
    fields[..., SIGMA] = u                              # field sigma(j) holds code j
    lo = np.zeros(u.shape[:-1], np.uint64)
    hi = np.zeros(u.shape[:-1], np.uint64)
    for p in range(16):
        f = fields[..., p].astype(np.uint64)
        b = 6 * p
        if b + 6 <= 64:
            lo |= f << np.uint64(b)
        elif b >= 64:
            hi |= f << np.uint64(b - 64)
        else:
            lo |= f << np.uint64(b)
            hi |= f >> np.uint64(64 - b)
    words = np.stack([(lo & np.uint64(0xFFFFFFFF)).astype(np.uint32), (lo >> np.uint64(32)).astype(np.uint32),
                      hi.astype(np.uint32)], axis=-1)
    return words.astype("<u4").view(np.uint8).reshape(-1)
