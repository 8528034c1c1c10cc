"""CPU pins of the host coder of the FP6 operand layout (tests/f6_layout.py)
against the layout's definition in include/libspin.h."""

import numpy as np

from tests import f6_layout


def test_round_trip_and_size():
    rng = np.random.default_rng(0)
    for M, K in [(1, 64), (33, 128), (70, 256)]:
        q = rng.integers(-8, 8, size=(M, K))
        buf = f6_layout.encode(q)
        assert buf.size == f6_layout.nbytes(M, K)
        assert np.array_equal(f6_layout.decode(buf, M, K), q)


def test_one_code_lands_where_the_definition_puts_it():
    """Row 33, column 100 of a 64 x 192 matrix: region (33 / 32) * 3 + 100 / 64 = 4,
    byte ((100 % 64) / 32) * 768 + (33 % 32) * 24 + ((100 % 32) / 16) * 12 = 792
    of it, field sigma(100 % 16 = 4) = 3, bits 18 .. 23."""
    M, K = 64, 192                        # whole row blocks: no padding rows
    q = np.full((M, K), -8)              # u = 0 everywhere: all-zero bytes
    q[33, 100] = 5                        # u = 13 = 0b1101
    buf = f6_layout.encode(q)
    nz = np.flatnonzero(buf)
    base = 4 * 1536 + 792
    bits = 13 << 18
    want = {base + i: (bits >> (8 * i)) & 0xFF for i in range(12) if (bits >> (8 * i)) & 0xFF}
    assert dict(zip(nz.tolist(), buf[nz].tolist())) == want


def test_sigma_is_a_permutation():
    assert sorted(f6_layout.SIGMA.tolist()) == list(range(16))
