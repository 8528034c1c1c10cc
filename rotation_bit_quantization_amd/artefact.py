"""Folded weights on disk: the persistent product of the offline fold
(page "SpinQuant, Reproduced", Q5: R1/R2 and R4's inverse are merged into
the weights once, then the weights are quantized per output channel).

A layer's folded weights are two numpy .npy files side by side:

    <stem>.codes.npy    uint8   [N, K/2]  packed INT4 codes as spin_fold_rotation
                                          writes them (two's complement, code k in
                                          the low nibble of byte k/2 when k is even)
    <stem>.scales.npy   float32 [N]       per-output-channel scales

Both are written and read with numpy's own array format and pickling
disabled, so loading a file executes nothing from it.  Loading checks dtype,
rank and that the two files agree on N; it never converts a value.
"""

import numpy as np
import torch

__all__ = ["save_folded", "load_folded", "folded_paths"]


def folded_paths(stem):
    """(codes path, scales path) for a stem."""
    return stem + ".codes.npy", stem + ".scales.npy"


def _host(a, dtype, ndim, name):
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    a = np.asarray(a)
    if a.dtype != dtype or a.ndim != ndim:
        raise ValueError(f"{name}: expected {np.dtype(dtype).name} of rank {ndim}, got {a.dtype} {a.shape}")
    return np.ascontiguousarray(a)


def save_folded(stem, Wq, w_scale):
    """Write packed codes Wq [N, K/2] uint8 and scales w_scale [N] float32
    (torch tensors on any device, or numpy arrays); returns the two paths."""
    codes = _host(Wq, np.uint8, 2, "Wq")
    scales = _host(w_scale, np.float32, 1, "w_scale")
    if codes.shape[0] != scales.shape[0]:
        raise ValueError(f"Wq has {codes.shape[0]} rows but w_scale {scales.shape[0]} entries")
    pc, ps = folded_paths(stem)
    np.save(pc, codes, allow_pickle=False)
    np.save(ps, scales, allow_pickle=False)
    return pc, ps


def load_folded(stem, device=None):
    """Read a pair written by save_folded; returns (Wq, w_scale) as torch
    tensors on `device` (host memory when None)."""
    pc, ps = folded_paths(stem)
    codes = np.load(pc, allow_pickle=False)
    scales = np.load(ps, allow_pickle=False)
    codes = _host(codes, np.uint8, 2, pc)
    scales = _host(scales, np.float32, 1, ps)
    if codes.shape[0] != scales.shape[0]:
        raise ValueError(f"{pc} has {codes.shape[0]} rows but {ps} {scales.shape[0]} entries")
    Wq, w_scale = torch.from_numpy(codes), torch.from_numpy(scales)
    if device is not None:
        Wq, w_scale = Wq.to(device), w_scale.to(device)
    return Wq, w_scale
