"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and arranges them into the shapes of
the workloads (Qwen3-8B sizes: hidden 4096, 32 heads x 128, MLP width 12288,
page "SpinQuant, Reproduced", Q5 figure caption).  It contains none of the
method's arithmetic: no Hadamard, no quantizer, no fold, no GEMM.  The only
linear algebra here builds inputs: a Haar-random orthogonal matrix (QR of a
Gaussian) and, for the R1-folded projection, the residual stream expressed in
the rotated basis (the stand-in for R1 having been folded upstream).

Every draw uses numpy's PCG64 ``default_rng(seed)``, in float64, in the order
outlier indices, activations, weights, rotation; casts to float16 / float32
happen once at the end.  The outlier recipe stands in for the real activation
statistics the pages measure (kurtosis in the hundreds before rotation,
page "SpinQuant, Reproduced", Q3).
"""

import numpy as np

__all__ = [
    "outlier_activations", "gaussian_weight", "haar_orthogonal", "kv_heads",
    "tiny_config", "down_config", "kv_config", "qkv_config", "chain_config", "probe_config",
    "r2_config",
]


def outlier_activations(rng, M, K, n_outliers, mult, dtype=np.float16, idx=None):
    """[M, K] N(0, 1) activations whose ``n_outliers`` channels are scaled by ``mult``.

    Channels are drawn with ``rng.choice(K, n_outliers, replace=False)`` unless
    ``idx`` is given.  Returns (x cast to ``dtype``, channel indices).
    """
    if idx is None:
        idx = rng.choice(K, size=n_outliers, replace=False) if n_outliers else np.zeros(0, np.int64)
    x = rng.standard_normal((M, K))
    if len(idx):
        x[:, idx] *= mult
    return x.astype(dtype), np.asarray(idx)


def gaussian_weight(rng, K, N, std=0.02):
    """[K, N] float32 weight drawn N(0, std^2) (std = 0.02)."""
    return (rng.standard_normal((K, N)) * std).astype(np.float32)


def haar_orthogonal(rng, n):
    """n x n float32 random orthogonal matrix: QR of a float64 Gaussian with the
    sign of R's diagonal moved into Q (making Q unique), then one cast to float32."""
    g = rng.standard_normal((n, n))
    q, r = np.linalg.qr(g)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return (q * d[None, :]).astype(np.float32)


def kv_heads(rng, T, H, D, n_out_per_head, mult, dtype=np.float16):
    """[T, H, D] N(0, 1) vectors; in each head ``n_out_per_head`` dims (drawn per
    head without replacement) are scaled by ``mult``."""
    idx = np.stack([rng.choice(D, size=n_out_per_head, replace=False) for _ in range(H)]) \
        if n_out_per_head else np.zeros((H, 0), np.int64)
    x = rng.standard_normal((T, H, D))
    for h in range(H):
        if idx.shape[1]:
            x[:, h, idx[h]] *= mult
    return x.astype(dtype)


# ---------------------------------------------------------------- workloads

def tiny_config(seed=1, M=64, K=256, N=256):
    """Tiny: X 64x256 fp32 with 4 outlier channels x50; Hadamard n = 256;
    W 256x256 N(0, 0.02); R a Haar rotation of order 256."""
    rng = np.random.default_rng(seed)
    x, idx = outlier_activations(rng, M, K, 4, 50.0, dtype=np.float32)
    w = gaussian_weight(rng, K, N)
    r = haar_orthogonal(rng, K)
    return {"x": x, "w": w, "r": r, "had_n": K, "outlier_idx": idx}


def down_config(seed=2, M=4096, K=12288, N=4096, x_dtype=np.float16):
    """R4 / down_proj: X MxK fp16 with round(0.1% K) outlier channels x100,
    Hadamard order K = 12 * 1024, W KxN N(0, 0.02) folded with R = None."""
    rng = np.random.default_rng(seed)
    n_out = int(round(0.001 * K))
    x, idx = outlier_activations(rng, M, K, n_out, 100.0, dtype=x_dtype)
    w = gaussian_weight(rng, K, N)
    return {"x": x, "w": w, "had_n": K, "outlier_idx": idx}


def kv_config(seed=3, T=4096, H=32, D=128):
    """R3 / KV: Q, K [T][H][D] fp16 with 2 outlier dims per head x30; V without outliers."""
    rng = np.random.default_rng(seed)
    q = kv_heads(rng, T, H, D, 2, 30.0)
    k = kv_heads(rng, T, H, D, 2, 30.0)
    v = kv_heads(rng, T, H, D, 0, 1.0)
    return {"q": q, "k": k, "v": v}


def qkv_config(seed=4, M=4096, K=4096, N=6144):
    """R1-folded qkv_proj: R1 Haar KxK; W KxN; residual X_out with 8 outlier
    channels x100, handed over as fp16(X_out . R1) (R1 folded upstream)."""
    rng = np.random.default_rng(seed)
    x_out, idx = outlier_activations(rng, M, K, 8, 100.0, dtype=np.float64)
    w = gaussian_weight(rng, K, N)
    r1 = haar_orthogonal(rng, K)
    x = (x_out @ r1.astype(np.float64)).astype(np.float16)
    return {"x": x, "x_out": x_out, "w": w, "r": r1, "had_n": 1, "outlier_idx": idx}


def chain_config(seed=5, M=8192, hidden=4096, heads=32, head_dim=128, mlp=12288):
    """Decoder-layer linear chain: qkv (N = 6144, R1), o_proj (4096^2, head-wise
    R2 of order 128), gate/up (N = 2 * 12288, R1), down (K = 12288, Hadamard).
    Activations N(0, 1) with 0.1% outlier channels x100, weights N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    out = {"M": M}
    layers = [
        ("qkv", hidden, hidden + 2 * 1024, "r1"),
        ("o", hidden, hidden, "r2"),
        ("gate_up", hidden, 2 * mlp, "r1"),
        ("down", mlp, hidden, None),
    ]
    r1 = None
    for name, K, N, rot in layers:
        n_out = int(round(0.001 * K))
        x, _ = outlier_activations(rng, M, K, n_out, 100.0, dtype=np.float16)
        w = gaussian_weight(rng, K, N)
        if rot == "r1":
            if r1 is None:
                r1 = haar_orthogonal(rng, hidden)
            r, r_block = r1, hidden
        elif rot == "r2":
            r, r_block = haar_orthogonal(rng, head_dim), head_dim
        else:
            r, r_block = None, K
        out[name] = {"x": x, "w": w, "r": r, "r_block": r_block,
                     "had_n": K if name == "down" else 1}
    return out


def probe_config(seed=6, T=2048, K=1024, N=1024, draws=32, n_outliers=8, mult=100.0):
    """Rotation-choice probe on one synthetic layer (page "SpinQuant,
    Reproduced", Q3: 32 randomised Hadamards against 32 random orthogonal
    matrices on one layer): activations T x K float32 with ``n_outliers``
    channels x ``mult``, weight K x N N(0, 0.02), ``draws`` Haar rotations of
    order K and ``draws`` vectors of K random signs (+1 / -1)."""
    rng = np.random.default_rng(seed)
    x, idx = outlier_activations(rng, T, K, n_outliers, mult, dtype=np.float32)
    w = gaussian_weight(rng, K, N)
    haar = [haar_orthogonal(rng, K) for _ in range(draws)]
    signs = [rng.choice(np.array([-1.0, 1.0], np.float32), size=K) for _ in range(draws)]
    return {"x": x, "w": w, "haar": haar, "signs": signs, "outlier_idx": idx}


def r2_config(seed=7, T=512, heads=32, head_dim=128, N=1024, draws=32, n_out_per_head=2, mult=30.0):
    """Learning R2 on one synthetic o_proj slice (page "SpinQuant, Reproduced",
    Q5: one 128 x 128 rotation shared by the 32 heads, learned against the
    layer's W4A4 output error, weights frozen): the value-path activations
    T x (heads * head_dim) float32 with ``n_out_per_head`` outlier dims per head
    x ``mult``, a weight (heads * head_dim) x N N(0, 0.02), and ``draws``
    vectors of head_dim random signs for the random-Hadamard baselines."""
    rng = np.random.default_rng(seed)
    x = kv_heads(rng, T, heads, head_dim, n_out_per_head, mult, dtype=np.float32).reshape(T, heads * head_dim)
    w = gaussian_weight(rng, heads * head_dim, N)
    signs = [rng.choice(np.array([-1.0, 1.0], np.float32), size=head_dim) for _ in range(draws)]
    return {"x": x, "w": w, "signs": signs, "heads": heads, "head_dim": head_dim}
