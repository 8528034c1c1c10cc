"""Diagnostics the pages report (oracle; test infrastructure).

Page "SpinQuant, Reproduced", Q3: kurtosis measures tailedness (a Gaussian
has 3); it is taken across the channels within one token and averaged over
tokens; the paper reports layers above 200 before rotation and about 3 after.
Reading: Pearson (non-excess) kurtosis with central moments,
m4 / m2^2, computed in float64.

Page "SpinQuant, Reproduced", Q6: the Cayley update keeps R orthogonal, and
the orthogonality error is the number to check; here max |R^T R - I|.
"""

import numpy as np

__all__ = ["kurtosis_per_token", "mean_kurtosis", "orthogonality_error"]


def kurtosis_per_token(x) -> np.ndarray:
    """Pearson kurtosis of each row (token) across its last axis (channels)."""
    x64 = np.asarray(x, dtype=np.float64)
    x64 = x64.reshape(-1, x64.shape[-1])
    c = x64 - x64.mean(axis=1, keepdims=True)
    m2 = np.mean(c * c, axis=1)
    m4 = np.mean(c ** 4, axis=1)
    return m4 / (m2 * m2)


def mean_kurtosis(x, max_tokens: int = 512) -> float:
    """Average per-token kurtosis over the first ``max_tokens`` rows."""
    x64 = np.asarray(x)
    x64 = x64.reshape(-1, x64.shape[-1])[:max_tokens]
    return float(np.mean(kurtosis_per_token(x64)))


def orthogonality_error(R) -> float:
    """max |R^T R - I| in float64."""
    R64 = np.asarray(R, dtype=np.float64)
    return float(np.max(np.abs(R64.T @ R64 - np.eye(R64.shape[0]))))
