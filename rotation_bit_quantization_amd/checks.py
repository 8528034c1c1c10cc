"""Cheap checks on rotation inputs (page "SpinQuant, Reproduced", Q5: the
Cayley form keeps a learned R orthogonal, and its orthogonality error is the
number to check; the same check applies to every R handed to the fold).

orthogonality_error(R) = max |R^T R - I| with R^T R formed on the device by
spin_fold_rotation itself (folding R into R: W' = R^T R, float32 accumulation)
and only the O(r^2) comparison done on the host.  With float32 accumulation
the error floor is about r * 2^-24 (1e-6 .. 3e-4 for r = 128 .. 4096), far
below what a non-orthogonal input shows.
"""

import numpy as np

from . import spin

__all__ = ["orthogonality_error"]


def orthogonality_error(R) -> float:
    """max |R^T R - I| for a float32 [r][r] device tensor R (r a multiple of 64)."""
    r = R.shape[0]
    if R.shape != (r, r) or r % 64 != 0:
        raise ValueError("R must be square with an order that is a multiple of 64")
    gram, _, _ = spin.spin_fold_rotation(R, R, r)
    g = gram.cpu().numpy().astype(np.float64)
    return float(np.abs(g - np.eye(r)).max())
