"""Cayley update of an orthogonal matrix (oracle; test infrastructure).

Page "SpinQuant, Reproduced", Q5 ("Cayley SGD keeps R orthogonal exactly"):
a plain gradient step would leave the orthogonal group, so the rotation is
updated by the Cayley transform of a skew-symmetric matrix Y,

    R' = (I - alpha/2 Y)^{-1} (I + alpha/2 Y) R,

which is orthogonal for every Y with Y^T = -Y.  The pages give the update but
not Y.  Reading taken here: Y = R G^T - G R^T with G the Euclidean gradient of
the loss at R, the skew matrix whose first-order step alpha Y R = alpha (R G^T R - G)
is the steepest descent direction within the tangent space (it lowers the
loss whenever G R^T is not symmetric).  Everything is float64; the solve is a
library linear solve.
"""

import numpy as np

__all__ = ["skew_descent", "cayley_step"]


def skew_descent(R, G) -> np.ndarray:
    """Y = R G^T - G R^T (skew-symmetric) for orthogonal R and gradient G."""
    R = np.asarray(R, np.float64)
    G = np.asarray(G, np.float64)
    return R @ G.T - G @ R.T


def cayley_step(R, G, alpha: float) -> np.ndarray:
    """One Cayley update R' = (I - alpha/2 Y)^{-1} (I + alpha/2 Y) R with Y = skew_descent(R, G)."""
    R = np.asarray(R, np.float64)
    Y = skew_descent(R, G)
    eye = np.eye(R.shape[0])
    return np.linalg.solve(eye - 0.5 * alpha * Y, (eye + 0.5 * alpha * Y) @ R)
