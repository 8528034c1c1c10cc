"""Hadamard matrices and the dense online rotation (oracle; test infrastructure).

Page "SpinQuant, Reproduced", section Q5 (Method 1/2): R3 (KV path) and R4
(before down_proj) cannot be folded into weights, so they run online and must
be a rotation that can be applied quickly, i.e. a Hadamard matrix.  The page
gives no construction.  Readings taken here:

  * power-of-two orders use Sylvester's construction in natural order,
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]  (equivalently
    H[i][j] = (-1)^popcount(i & j));
  * order 12 uses Paley's first construction with the field GF(11);
  * orders 12 * 2^k use the Kronecker product H_12 (x) H_{2^k}; element
    index i = a * 2^k + b with a the H_12 index;
  * the rotation is the normalised matrix H / sqrt(n), applied to a row vector
    from the right, y = x . (H / sqrt(n)), block-diagonally along the row when
    n is smaller than the row length.

Everything is built from those definitions; no fast transform is used here.
The rotation is a dense float64 product (``x @ H``), divided by sqrt(n) in
float64, and the caller rounds the float64 result once to float32.
"""

import functools

import numpy as np

__all__ = ["sylvester", "paley12", "hadamard", "rotate_rows", "supported_had_n"]


def sylvester(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), int64, natural order.

    Built by the doubling recursion H_2m = [[H_m, H_m], [H_m, -H_m]] starting
    from H_1 = [1].
    """
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"Sylvester order must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _quadratic_character_mod(q: int) -> np.ndarray:
    """chi[x] for x in 0..q-1: 0 at 0, +1 on nonzero squares mod q, -1 otherwise."""
    squares = {(x * x) % q for x in range(1, q)}
    chi = np.full(q, -1, dtype=np.int64)
    chi[0] = 0
    for s in squares:
        chi[s] = 1
    return chi


def paley12() -> np.ndarray:
    """Order-12 Hadamard matrix from Paley's first construction over GF(11).

    Jacobsthal matrix Q[a][b] = chi(b - a) (chi = quadratic character mod 11),
    conference matrix S = [[0, 1^T], [-1, Q]] (border row of +1, border column
    of -1), and H = I + S.  Row and column 0 are the border; rows 1..11 are the
    field elements 0..10.  Since 11 = 3 mod 4, Q is skew, so S is skew and
    H + H^T = 2 I while H H^T = 12 I.
    """
    q = 11
    chi = _quadratic_character_mod(q)
    jac = np.empty((q, q), dtype=np.int64)
    for a in range(q):
        for b in range(q):
            jac[a, b] = chi[(b - a) % q]
    s = np.zeros((q + 1, q + 1), dtype=np.int64)
    s[0, 1:] = 1
    s[1:, 0] = -1
    s[1:, 1:] = jac
    return np.eye(q + 1, dtype=np.int64) + s


def supported_had_n(n: int) -> bool:
    """Orders the library supports: 1, 2^k (1 <= k <= 14), 12 * 2^k (0 <= k <= 10)."""
    if n == 1:
        return True
    if n >= 2 and (n & (n - 1)) == 0 and n <= (1 << 14):
        return True
    if n >= 12 and n % 12 == 0:
        m = n // 12
        return (m & (m - 1)) == 0 and m <= (1 << 10)
    return False


@functools.lru_cache(maxsize=8)
def hadamard(n: int) -> np.ndarray:
    """Unnormalised Hadamard matrix of order n used by the library (int64, read-only)."""
    if not supported_had_n(n):
        raise ValueError(f"unsupported Hadamard order {n}")
    if n == 1:
        h = np.ones((1, 1), dtype=np.int64)
    elif (n & (n - 1)) == 0:
        h = sylvester(n)
    else:
        h = np.kron(paley12(), sylvester(n // 12))
    h.setflags(write=False)
    return h


def rotate_rows(x, n: int) -> np.ndarray:
    """Exact-as-float64 rotation y = x . blockdiag(H_n / sqrt(n), ...) of each row.

    ``x`` is any real array of shape [..., K] with K a multiple of n; it is
    converted to float64 (fp16 / fp32 inputs convert exactly).  Each length-n
    block of a row is multiplied densely by H_n and divided by sqrt(n).
    Returns float64 of the same shape; callers round once to float32.
    """
    x64 = np.asarray(x, dtype=np.float64)
    k = x64.shape[-1]
    if k % n != 0:
        raise ValueError(f"row length {k} is not a multiple of the Hadamard order {n}")
    if n == 1:
        return x64.copy()
    h = hadamard(n).astype(np.float64)
    blocks = x64.reshape(-1, n)
    y = (blocks @ h) / np.sqrt(np.float64(n))
    return y.reshape(x64.shape)
