"""Learning the head-wise rotation R2 with Cayley SGD (offline, upstream of
the fold; page "SpinQuant, Reproduced", Q5).

R2 is one orthogonal head_dim x head_dim matrix shared by all heads of a
layer's value path; it is folded into the value and output projections, so
the layer computes (x B)(B^T w) with B = blockdiag(R2, ..., R2) and the
full-precision output is unchanged.  Quantized, the output error depends on
R2, and R2 is learned against it with the weights frozen:

  * objective: the layer's W4A4 relative output error,
        L(R2) = ||Q(x B) Q(B^T w) - x w||_F^2 / ||x w||_F^2,
    Q the per-token / per-output-channel absmax INT4 quantizer;
  * round() has zero gradient almost everywhere, so it is passed straight
    through (its gradient taken as 1) - without that the loss carries no
    signal back to R2; the absmax scales are differentiated as they are (the
    gradient of a maximum reaches its largest element), which is what lets a
    rotation lower each token's and each channel's maximum relative to the
    rest;
  * update: the Cayley transform R2' = (I - a/2 Y)^{-1} (I + a/2 Y) R2 with
    Y = R2 G^T - G R2^T (G the gradient), orthogonal for every step size;
    the step size a = lr / ||Y||_F fixes the length of each step.

The gradient runs on the host in float64 (PyTorch autograd on the CPU, as
the pages' own run does); the error that is reported is measured on the
device through libspin: fold of the activations and of the weight with
blockdiag(R2), then the W4A4 GEMM.

    python -m rotation_bit_quantization_amd.cayley [--iters 120] [--lr 0.2]
"""

import argparse
import json
import time

import numpy as np
import torch

from . import probe, spin, synth

__all__ = ["cayley_update", "ste_layer_loss", "learn_r2", "r2_experiment"]


def cayley_update(R, G, alpha):
    """R' = (I - alpha/2 Y)^{-1} (I + alpha/2 Y) R with Y = R G^T - G R^T (torch, any float dtype)."""
    Y = R @ G.T - G @ R.T
    eye = torch.eye(R.shape[0], dtype=R.dtype, device=R.device)
    return torch.linalg.solve(eye - 0.5 * alpha * Y, (eye + 0.5 * alpha * Y) @ R)


class _RoundSTE(torch.autograd.Function):
    """Round half to even forward, identity backward (straight-through)."""

    @staticmethod
    def forward(ctx, v):
        return torch.round(v)

    @staticmethod
    def backward(ctx, g):
        return g


def _quant_ste(v, dim):
    s = v.abs().amax(dim=dim, keepdim=True) / 7.0
    s = torch.where(s == 0, torch.ones_like(s), s)
    return torch.clamp(_RoundSTE.apply(v / s), -7.0, 7.0) * s


def ste_layer_loss(x, w, r2, heads):
    """L(R2) above for x [T, heads * d], w [heads * d, N], r2 [d, d] (torch tensors)."""
    T, d, N = x.shape[0], r2.shape[0], w.shape[1]
    xr = (x.reshape(T, heads, d) @ r2).reshape(T, heads * d)
    wr = (r2.T @ w.reshape(heads, d, N)).reshape(heads * d, N)
    y = _quant_ste(xr, 1) @ _quant_ste(wr, 0)
    ref = x @ w
    return ((y - ref) ** 2).sum() / (ref ** 2).sum()


def learn_r2(x, w, r_init, heads, iters=120, lr=0.2):
    """Cayley SGD on R2 from ``r_init``; returns (R2 float64 numpy, loss history)."""
    xt = torch.as_tensor(np.asarray(x, np.float64))
    wt = torch.as_tensor(np.asarray(w, np.float64))
    R = torch.as_tensor(np.asarray(r_init, np.float64)).clone()
    hist = []
    for _ in range(iters):
        R.requires_grad_(True)
        loss = ste_layer_loss(xt, wt, R, heads)
        (G,) = torch.autograd.grad(loss, R)
        hist.append(loss.item())
        with torch.no_grad():
            Y = R @ G.T - G @ R.T
            nrm = float(torch.linalg.norm(Y))
            R = cayley_update(R.detach(), G, lr / nrm if nrm > 0 else 0.0)
    return np.ascontiguousarray(R.numpy()), hist


def r2_experiment(cfg=None, iters=120, lr=0.2, device="cuda"):
    """The 32 random Hadamards diag(s) H_d / sqrt(d) against the R2 learned
    from the best of them; errors measured through libspin."""
    cfg = synth.r2_config() if cfg is None else cfg
    x, w, heads, d = cfg["x"], cfg["w"], cfg["heads"], cfg["head_dim"]
    y_ref = x.astype(np.float64) @ w.astype(np.float64)
    xd, wd = torch.from_numpy(x).to(device), torch.from_numpy(w).to(device)
    h = probe.library_hadamard(d, device).cpu().numpy()
    draws = [np.ascontiguousarray(s[:, None] * h) for s in cfg["signs"]]
    errs = [probe.w4a4_layer_error(xd, wd, torch.from_numpy(r).to(device), y_ref)[0] for r in draws]
    best = int(np.argmin(errs))
    t0 = time.perf_counter()
    # float64 start: the draw's signs over sqrt(d) (its float32 entries are
    # rounded, which the Cayley steps would otherwise carry along)
    r0 = np.sign(draws[best].astype(np.float64)) / np.sqrt(np.float64(d))
    R, hist = learn_r2(x, w, r0, heads, iters, lr)
    t_learn = time.perf_counter() - t0
    R32 = np.ascontiguousarray(R, dtype=np.float32)
    learned = probe.w4a4_layer_error(xd, wd, torch.from_numpy(R32).to(device), y_ref)[0]
    return {
        "workload": {"tokens": int(x.shape[0]), "heads": heads, "head_dim": d, "out": int(w.shape[1]),
                     "iters": iters, "lr": lr},
        "random_hadamard": {"min": float(min(errs)), "max": float(max(errs)), "mean": float(np.mean(errs))},
        "learned": learned,
        "gain_vs_best_draw": 1.0 - learned / min(errs),
        "orthogonality_error": float(np.abs(R.T @ R - np.eye(d)).max()),
        "orthogonality_error_fp32": float(np.abs(R32.astype(np.float64).T @ R32 - np.eye(d)).max()),
        "ste_loss_first_last": [hist[0], hist[-1]],
        "host_seconds_per_iter": t_learn / max(1, iters),
        "R2": R32,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--iters", type=int, default=120)
    ap.add_argument("--lr", type=float, default=0.2)
    a = ap.parse_args()
    res = r2_experiment(iters=a.iters, lr=a.lr)
    res.pop("R2")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
