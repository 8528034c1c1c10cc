"""GPU parity of the W4A4 GEMM on the FP6 matrix cores (K from 256 to 65536),
whole and with K split into slices.

The codes enter the block-scaled FP6 MFMA as u = q + 8, the float32
accumulator holds sum u_a u_b exactly while 225 K < 2^24, and the epilogue
subtracts the code sums; the int32 accumulators must equal the oracle's
int64 product bit for bit, the outputs the oracle epilogue on them.  The
cases cover ragged M and N (rows and columns past the last full tile), the
largest K the path takes with every code at +-7 and with -8 nibbles (u = 0,
accepted by the ABI), and the first K past the limit (the int8 kernels).
The split-K form adds each slice's exact int32 partial into the output and
dequantizes in a last pass: the same bits as the whole-K kernels.
"""

import numpy as np
import pytest
import torch

import oracle  # noqa: F401  (the oracle behind check_gemm)
from rotation_bit_quantization_amd import spin
from tests.test_gpu_parity import DEV, _dev, _host, check_gemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spin.load()


def _codes(M, N, K, seed):
    rng = np.random.default_rng(seed)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    return qx, qw, sx, sw


@pytest.mark.parametrize("M,N,K", [(17, 5, 8192), (37, 53, 8192), (257, 300, 8192), (300, 200, 12288),
                                   (600, 1000, 16384), (4096 + 37, 256 + 3, 12288), (1000, 1030, 8320),
                                   (1, 1, 256), (40, 70, 384), (33, 300, 640), (300, 31, 4096)])
def test_gemm_fp6_ragged(M, N, K):
    """The FP6 kernel named explicitly: ragged tiles, the shortest pipelines
    (two and three steps of 128 codes) and odd step counts; its outputs must
    also equal the int8 kernels' bit for bit."""
    qx, qw, sx, sw = _codes(M, N, K, M * 31 + N + K)
    y6, a6 = check_gemm(qx, qw, sx, sw, kernel=spin.SPIN_GEMM_FP6)
    y8, a8 = check_gemm(qx, qw, sx, sw, kernel=spin.SPIN_GEMM_INT8)
    assert np.array_equal(a6, a8) and np.array_equal(y6, y8)


def test_gemm_auto_matches_both_families():
    """The automatic choice (the FP6 kernel at this shape) gives the same bits."""
    qx, qw, sx, sw = _codes(1024, 1024 + 64, 8192, 7)
    y, a = check_gemm(qx, qw, sx, sw, rows=np.arange(0, 1024, 9))
    y6, a6 = check_gemm(qx, qw, sx, sw, rows=[0], kernel=spin.SPIN_GEMM_FP6)
    assert np.array_equal(a, a6) and np.array_equal(y, y6)


def test_gemm_fp6_k_outside_its_range():
    qx, qw, sx, sw = _codes(4, 4, 128, 1)
    with pytest.raises(spin.SpinError) as e:
        check_gemm(qx, qw, sx, sw, kernel=spin.SPIN_GEMM_FP6)
    assert e.value.status == spin.SPIN_ERR_BAD_SHAPE


@pytest.mark.parametrize("K,kernel", [(65536, "fp6"), (65536, "auto"), (65536 + 128, "auto")])
def test_gemm_fp6_largest_k_extremes(K, kernel):
    """K = 65536 is the largest the FP6 kernel takes (225 K < 2^24); every code +-7
    gives |acc| = 49 K, -8 nibbles give u = 0 against u = 15; one more step
    runs the int8 kernels."""
    M, N = 20, 7
    rng = np.random.default_rng(K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qx[0] = 7
    qx[1] = -7
    qx[2] = -8                                   # u = 0
    qx[3, ::2] = -8
    qx[3, 1::2] = 7
    qw[0] = 7                                    # u = 15
    qw[1] = -7
    qw[2] = -8
    kern = spin.SPIN_GEMM_FP6 if kernel == "fp6" else None
    _, a = check_gemm(qx, qw, np.ones(M, np.float32), np.ones(N, np.float32), kernel=kern)
    assert a[0, 0] == 49 * K and a[1, 0] == -49 * K and a[0, 1] == -49 * K
    assert a[2, 2] == 64 * K and a[2, 0] == -56 * K


# ---------------------------------------------------------------- split K

@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (37, 53, 8320), (300, 200, 12288), (257, 300, 16384),
                                   (1000, 1030, 8320), (4096 + 37, 259, 12288), (300, 31, 4096),
                                   (129, 4096 + 16, 384), (200, 600, 32768)])
def test_gemm_fp6_splitk_ragged(M, N, K):
    """The split-K form named explicitly: one slice (two and three steps),
    slices of two or three steps (65 steps over 32 slices), ragged tiles and
    slice counts that do not divide the steps; all rows against the oracle
    and every bit equal to the int8 kernels'."""
    qx, qw, sx, sw = _codes(M, N, K, M * 13 + N + K)
    ys, as_ = check_gemm(qx, qw, sx, sw, kernel=spin.SPIN_GEMM_FP6_SPLITK)
    y8, a8 = check_gemm(qx, qw, sx, sw, rows=[0], kernel=spin.SPIN_GEMM_INT8)
    assert np.array_equal(as_, a8) and np.array_equal(ys.view(np.uint32), y8.view(np.uint32))


@pytest.mark.parametrize("M,N", [(129, 4096), (256, 4096), (512, 4096 + 64), (1000, 4096), (1024, 2048)])
def test_gemm_auto_mid_size_rows(M, N):
    """129 to 1024 rows at K = 12288: the sizes AUTO takes through split K.
    Sampled rows from every row block against the oracle, every output equal
    to the unsplit FP6 kernel's and the int8 kernels' bits."""
    K = 12288
    qx, qw, sx, sw = _codes(M, N, K, M + N)
    rows = np.unique(np.linspace(0, M - 1, 24).astype(int))
    y, a = check_gemm(qx, qw, sx, sw, rows=rows)
    for kern in (spin.SPIN_GEMM_FP6, spin.SPIN_GEMM_INT8):
        y2, a2 = check_gemm(qx, qw, sx, sw, rows=[M - 1], kernel=kern)
        assert np.array_equal(a, a2) and np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_gemm_splitk_largest_k_extremes():
    """K = 65536 split into slices: every slice's partial at the +-7 and -8
    extremes, summed into |acc| = 49 K and 64 K exactly."""
    K, M, N = 65536, 20, 7
    rng = np.random.default_rng(K + 1)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qx[0], qx[1], qx[2] = 7, -7, -8
    qw[0], qw[1], qw[2] = 7, -7, -8
    _, a = check_gemm(qx, qw, np.ones(M, np.float32), np.ones(N, np.float32), kernel=spin.SPIN_GEMM_FP6_SPLITK)
    assert a[0, 0] == 49 * K and a[1, 0] == -49 * K and a[0, 1] == -49 * K
    assert a[2, 2] == 64 * K and a[2, 0] == -56 * K


def test_gemm_splitk_overwrites_and_replays_in_a_graph():
    """The split form's three launches (zero fill, slices, dequantizing pass)
    on outputs that held NaN and junk, then captured in a graph and replayed
    four times with eager writes to the outputs in between: every replay the
    eager bits."""
    M, N, K = 384, 1536, 8192
    qx, qw, sx, sw = _codes(M, N, K, 77)
    Xq, Wq = _dev(oracle.pack_int4(qx)), _dev(oracle.pack_int4(qw))
    xs, ws = _dev(sx), _dev(sw)
    Y = torch.full((M, N), float("nan"), device=DEV)
    acc = torch.full((M, N), -12345, dtype=torch.int32, device=DEV)

    def run():
        spin.spin_w4a4_gemm(Xq, xs, Wq, ws, Y=Y, acc_out=acc, kernel=spin.SPIN_GEMM_FP6_SPLITK)

    run()
    y, a = _host(Y).copy(), _host(acc).copy()
    rows = np.arange(0, M, 37)
    a_ref = oracle.gemm_rows(qx, qw, rows)
    assert np.array_equal(a[rows].astype(np.int64), a_ref)
    assert np.array_equal(y[rows], oracle.dequant(a_ref, sx[rows], sw))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        run()
    for rep in range(4):
        Y.fill_(float("nan"))
        acc.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        assert np.array_equal(_host(Y).view(np.uint32), y.view(np.uint32)), f"replay {rep}: Y"
        assert np.array_equal(_host(acc), a), f"replay {rep}: acc"
