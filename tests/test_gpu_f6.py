"""GPU parity of the FP6-operand-layout pair, through the C ABI:
spin_fwht_quant_f6 (R4 FWHT + per-token INT4, page "SpinQuant, Reproduced",
Q5, with the codes written in the FP6 operand layout of include/libspin.h)
and spin_w4a4_gemm_f6 (the W4A4 product on those codes).

Acceptance: the decoded codes (host decoder written from the layout's
definition, tests/f6_layout.py) and the scales are the bytes spin_fwht_quant
writes; x_sum is the sum of each row's codes; the GEMM's int32 accumulators
equal the oracle's int64 product and Y the oracle epilogue on them, and both
equal spin_w4a4_gemm's bits on the same codes.
"""

import numpy as np
import pytest
import torch

import oracle
from rotation_bit_quantization_amd import spin, synth
from tests import f6_layout

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spin.load()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _activations(M, seed):
    rng = np.random.default_rng(seed)
    x, _ = synth.outlier_activations(rng, M, 12288, 12, 100.0)
    if M > 3:
        x[3] = (x[3].astype(np.float32) * 1e-4).astype(np.float16)   # small row: the rescaled pass
    if M > 5:
        x[5] = 0                                                      # zero row: scale 0, codes 0
    return x


@pytest.mark.parametrize("M", [1, 37, 300, 4133])
def test_fwht_quant_f6_is_fwht_quant_in_the_layout(M):
    X = _dev(_activations(M, M))
    Xq, xs, _ = spin.spin_fwht_quant(X, 12288)
    Xf6, xsum, xs6 = spin.spin_fwht_quant_f6(X)
    codes = oracle.unpack_int4(_host(Xq))
    assert np.array_equal(f6_layout.decode(_host(Xf6), M, 12288), codes)
    assert np.array_equal(_host(xs6).view(np.uint32), _host(xs).view(np.uint32))
    assert np.array_equal(_host(xsum), codes.astype(np.int64).sum(axis=1))


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("M,K", [(1, 256), (37, 640), (300, 4096), (65, 12288), (33, 16384), (4133, 4096)])
def test_quant_only_f6_is_fwht_quant_in_the_layout(M, K, dtype):
    """had_n = 1: the codes and scales spin_fwht_quant(X, 1) writes (and the
    oracle's, quant-only being exact), in the layout, with their row sums;
    the both-FP6 GEMM on them gives the nibble GEMM's bits."""
    rng = np.random.default_rng(M + K)
    x = (rng.standard_normal((M, K)) * np.where(rng.random(K) < 0.002, 100.0, 1.0)).astype(dtype)
    if M > 3:
        x[3] *= dtype(1e-3)           # small row
    if M > 5:
        x[5] = 0                      # zero row: scale 0, codes 0
    if M > 7:                         # values on the rounding ties of their own scale
        x[7] = 0
        x[7, :14] = (np.arange(14) - 6.5).astype(dtype)   # absmax 7: s = 1, y / s = k + 1/2
        x[7, 15] = 7
    X = _dev(x)
    Xq, xs, _ = spin.spin_fwht_quant(X, 1)
    Xf6, xsum, xs6 = spin.spin_fwht_quant_f6(X, had_n=1)
    codes = oracle.unpack_int4(_host(Xq))
    assert np.array_equal(f6_layout.decode(_host(Xf6), M, K), codes)
    assert np.array_equal(_host(xs6).view(np.uint32), _host(xs).view(np.uint32))
    assert np.array_equal(_host(xsum), codes.astype(np.int64).sum(axis=1))
    pk, s_o, _ = oracle.fwht_quant(x, 1)
    assert np.array_equal(_host(Xq), pk) and np.array_equal(_host(xs), s_o)
    N = 96
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int64)
    Wq = _dev(oracle.pack_int4(qw))
    sw = _dev((rng.random(N) * 0.01).astype(np.float32))
    Wf6, wsum = spin.spin_codes_f6(Wq)
    Y6, acc6 = spin.spin_w4a4_gemm_f6f6(Xf6, xsum, xs6, Wf6, wsum, sw, K, want_acc=True)
    Y, acc = spin.spin_w4a4_gemm(Xq, xs, Wq, sw, want_acc=True)
    assert np.array_equal(_host(acc6), _host(acc))
    assert np.array_equal(_host(Y6).view(np.uint32), _host(Y).view(np.uint32))


def check_gemm_f6(qx, qw, sx, sw, rows=None):
    M, K = qx.shape
    Xf6 = _dev(f6_layout.encode(qx))
    xsum = _dev(qx.astype(np.int64).sum(axis=1).astype(np.int32))
    Wq = _dev(oracle.pack_int4(qw))
    Y, acc = spin.spin_w4a4_gemm_f6(Xf6, xsum, _dev(sx), Wq, _dev(sw), want_acc=True)
    y, a = _host(Y), _host(acc)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    a_ref = oracle.gemm_rows(qx, qw, sel)
    assert np.array_equal(a[sel].astype(np.int64), a_ref)
    assert np.array_equal(y[sel], oracle.dequant(a_ref, sx[sel], sw))
    Y2, acc2 = spin.spin_w4a4_gemm(_dev(oracle.pack_int4(qx)), _dev(sx), Wq, _dev(sw), want_acc=True)
    assert np.array_equal(_host(acc2), a) and np.array_equal(_host(Y2).view(np.uint32), y.view(np.uint32))
    Y3, _ = spin.spin_w4a4_gemm_f6(Xf6, xsum, _dev(sx), Wq, _dev(sw))
    assert np.array_equal(_host(Y3).view(np.uint32), y.view(np.uint32))
    return y, a


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (37, 53, 384), (40, 70, 640), (300, 200, 8192),
                                   (257, 300, 12288), (4096 + 37, 259, 12288), (1000, 1030, 8320)])
def test_gemm_f6_ragged(M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm_f6(qx, qw, sx, sw)


def test_gemm_f6_largest_k_extremes():
    """K = 65536 (the FP6 range's end) with every code at +-7 and -8 nibbles:
    |acc| = 49 K, u = 0 against u = 15."""
    K, M, N = 65536, 20, 7
    rng = np.random.default_rng(K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qx[0] = 7
    qx[1] = -7
    qx[2] = -8
    qw[0] = 7
    qw[1] = -7
    qw[2] = -8
    _, a = check_gemm_f6(qx, qw, np.ones(M, np.float32), np.ones(N, np.float32))
    assert a[0, 0] == 49 * K and a[1, 0] == -49 * K and a[0, 1] == -49 * K
    assert a[2, 2] == 64 * K and a[2, 0] == -56 * K


def test_down_proj_step_f6_full_size():
    """The down_proj workload through the pair equals the nibble pair bit for bit."""
    cfg = synth.down_config()
    X = _dev(cfg["x"])
    _, Wq, ws = spin.spin_fold_rotation(_dev(cfg["w"]), None, 12288)
    Xq, xs, _ = spin.spin_fwht_quant(X, 12288)
    Y, acc = spin.spin_w4a4_gemm(Xq, xs, Wq, ws, want_acc=True)
    Xf6, xsum, xs6 = spin.spin_fwht_quant_f6(X)
    Y6, acc6 = spin.spin_w4a4_gemm_f6(Xf6, xsum, xs6, Wq, ws, want_acc=True)
    assert np.array_equal(_host(acc6), _host(acc))
    assert np.array_equal(_host(Y6).view(np.uint32), _host(Y).view(np.uint32))


# ---------------------------------------------------------------- weights in the FP6 layout too

@pytest.mark.parametrize("N,K", [(1, 64), (37, 256), (300, 4096), (4096 + 5, 12288)])
def test_codes_f6_is_the_layout_of_the_codes(N, K):
    """spin_codes_f6 writes the weight codes in the FP6 operand layout (decoded
    by the host decoder written from the layout's definition) and their row sums."""
    rng = np.random.default_rng(N + K)
    qw = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    Wf6, wsum = spin.spin_codes_f6(_dev(oracle.pack_int4(qw)))
    assert np.array_equal(f6_layout.decode(_host(Wf6), N, K), qw)
    assert np.array_equal(_host(wsum), qw.astype(np.int64).sum(axis=1))


def check_gemm_f6f6(qx, qw, sx, sw, rows=None):
    M, K = qx.shape
    Xf6 = _dev(f6_layout.encode(qx))
    xsum = _dev(qx.astype(np.int64).sum(axis=1).astype(np.int32))
    Wq = _dev(oracle.pack_int4(qw))
    Wf6, wsum = spin.spin_codes_f6(Wq)
    Y, acc = spin.spin_w4a4_gemm_f6f6(Xf6, xsum, _dev(sx), Wf6, wsum, _dev(sw), K, want_acc=True)
    y, a = _host(Y), _host(acc)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    a_ref = oracle.gemm_rows(qx, qw, sel)
    assert np.array_equal(a[sel].astype(np.int64), a_ref)
    assert np.array_equal(y[sel], oracle.dequant(a_ref, sx[sel], sw))
    Y2, acc2 = spin.spin_w4a4_gemm(_dev(oracle.pack_int4(qx)), _dev(sx), Wq, _dev(sw), want_acc=True)
    assert np.array_equal(_host(acc2), a) and np.array_equal(_host(Y2).view(np.uint32), y.view(np.uint32))
    Y3, _ = spin.spin_w4a4_gemm_f6f6(Xf6, xsum, _dev(sx), Wf6, wsum, _dev(sw), K)
    assert np.array_equal(_host(Y3).view(np.uint32), y.view(np.uint32))
    return y, a


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (37, 53, 384), (40, 70, 640), (300, 200, 8192),
                                   (257, 300, 12288), (4096 + 37, 259, 12288), (1000, 1030, 8320)])
def test_gemm_f6f6_ragged(M, N, K):
    """Both operands copied into the stages: ragged tiles (the last 32-row
    blocks of both operands hold padding), the shortest pipelines (two and
    three steps) and odd step counts."""
    rng = np.random.default_rng(M * 5 + N + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm_f6f6(qx, qw, sx, sw)


def test_gemm_f6f6_largest_k_extremes():
    """K = 65536 with every code at +-7 and -8 nibbles."""
    K, M, N = 65536, 20, 7
    rng = np.random.default_rng(K + 2)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qx[0], qx[1], qx[2] = 7, -7, -8
    qw[0], qw[1], qw[2] = 7, -7, -8
    _, a = check_gemm_f6f6(qx, qw, np.ones(M, np.float32), np.ones(N, np.float32))
    assert a[0, 0] == 49 * K and a[1, 0] == -49 * K and a[0, 1] == -49 * K
    assert a[2, 2] == 64 * K and a[2, 0] == -56 * K


def test_down_proj_step_f6f6_full_size():
    """The down_proj workload with both operands in the FP6 layout equals the
    nibble path bit for bit."""
    cfg = synth.down_config()
    X = _dev(cfg["x"])
    _, Wq, ws = spin.spin_fold_rotation(_dev(cfg["w"]), None, 12288)
    Xq, xs, _ = spin.spin_fwht_quant(X, 12288)
    Y, acc = spin.spin_w4a4_gemm(Xq, xs, Wq, ws, want_acc=True)
    Xf6, xsum, xs6 = spin.spin_fwht_quant_f6(X)
    Wf6, wsum = spin.spin_codes_f6(Wq)
    Y6, acc6 = spin.spin_w4a4_gemm_f6f6(Xf6, xsum, xs6, Wf6, wsum, ws, 12288, want_acc=True)
    assert np.array_equal(_host(acc6), _host(acc))
    assert np.array_equal(_host(Y6).view(np.uint32), _host(Y).view(np.uint32))
