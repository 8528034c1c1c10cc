"""GPU parity: libspin (through its C ABI) against the CPU oracle.

Acceptance, per operation:
  * rotated float32 values (X_rot, W_rot) within 1e-5 relative of the oracle's
    float64 product, per row: ||d||_2 <= 1e-5 ||ref||_2 and
    max |d| <= 1e-5 max |ref|;
  * codes and scales bit-exact with the oracle quantizer applied to the GPU's
    own float32 rotated values (float32 decides the integer on both sides);
  * int32 accumulators bit-exact with the oracle's int64 GEMM;
  * final float32 outputs within 1e-3 relative of the oracle end to end, and
    bit-exact with the oracle epilogue applied to the GPU's accumulators.
"""

import numpy as np
import pytest
import torch

import oracle
from rotation_bit_quantization_amd import spin, synth

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


def assert_rows_close(got, ref, tol=1e-5):
    got = np.asarray(got, np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    d = got - ref
    nref = np.linalg.norm(ref, axis=1)
    assert (np.linalg.norm(d, axis=1) <= tol * nref + 1e-30).all(), \
        f"normwise rel err {np.max(np.linalg.norm(d, axis=1) / np.maximum(nref, 1e-30)):.3g}"
    assert (np.abs(d).max(axis=1) <= tol * np.abs(ref).max(axis=1) + 1e-30).all(), \
        f"max abs err {np.abs(d).max():.3g}"


def assert_y_close(got, ref, tol=1e-3, flip_rows=(), flip_cols=()):
    """Final outputs against the oracle's own end-to-end chain: per row
    ||d||_2 <= tol ||ref||_2, and |d| <= tol (|ref| + rms_row(ref)) for every
    element except those whose row or column holds a code that legitimately
    differs at a near-tie (the oracle rounds its float64 rotation, the GPU its
    float32 one); such flips are passed in and must themselves be rare."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    assert (np.linalg.norm(d, axis=1) <= tol * np.linalg.norm(ref, axis=1) + 1e-30).all()
    bad = np.abs(d) > tol * (np.abs(ref) + rms) + 1e-30
    explained = np.zeros_like(bad)
    explained[list(flip_rows), :] = True
    explained[:, list(flip_cols)] = True
    assert not (bad & ~explained).any(), f"{int((bad & ~explained).sum())} unexplained outliers"


def code_flips(gpu_packed, ref_packed, axis):
    """Indices (rows of a [R][K/2] code matrix) where GPU and oracle codes differ."""
    g = oracle.unpack_int4(gpu_packed)
    r = oracle.unpack_int4(ref_packed)
    diff = g != r
    assert diff.mean() < 1e-4, f"code mismatch rate {diff.mean()}"
    return np.nonzero(diff.any(axis=axis))[0]


def check_fwht_quant(x, had_n, rows=None):
    """Run spin_fwht_quant on x; check against the oracle on `rows` (all if None)."""
    X = _dev(x)
    Xq, xs, Xr = spin.spin_fwht_quant(X, had_n, want_rot=True)
    Xq2, xs2, _ = spin.spin_fwht_quant(X, had_n)                 # no X_rot: same codes
    xq, s, xr = _host(Xq), _host(xs), _host(Xr)
    assert np.array_equal(xq, _host(Xq2)) and np.array_equal(s, _host(xs2))
    # codes / scales: bit-exact with the oracle quantizer on the GPU's own y (all rows)
    c_ref, s_ref = oracle.quantize_rows(xr)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(xq, oracle.pack_int4(c_ref))
    # y against the oracle's float64 rotation (sampled rows at large sizes)
    sel = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    pk, s_o, y_o = oracle.fwht_quant(x[sel], had_n)
    assert_rows_close(xr[sel], y_o)
    mism = np.mean(oracle.unpack_int4(xq[sel]) != oracle.unpack_int4(pk))
    assert mism < 1e-4, f"direct code mismatch rate {mism}"
    return xq, s, xr


# ---------------------------------------------------------------- fwht_quant

def test_fwht_quant_tiny_config():
    cfg = synth.tiny_config()
    check_fwht_quant(cfg["x"], cfg["had_n"])


@pytest.mark.parametrize("had_n,K", [(1, 96), (2, 64), (16, 256), (128, 4096), (256, 768),
                                     (1024, 2048), (4096, 4096), (16384, 16384), (12, 96),
                                     (24, 480), (96, 192), (192, 3072), (3072, 6144),
                                     (12288, 12288), (12288, 24576)])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_fwht_quant_orders(had_n, K, dtype):
    rng = np.random.default_rng(had_n * 7 + K)
    M = 37
    x, _ = synth.outlier_activations(rng, M, K, max(1, K // 1000), 100.0, dtype=dtype)
    check_fwht_quant(x, had_n)


@pytest.mark.parametrize("K", [32, 2048, 2080, 4096, 12288, 16384, 32768])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_fwht_quant_quant_only(K, dtype):
    """had_n = 1 (rows already in the rotated basis): per-token INT4 only."""
    rng = np.random.default_rng(K + 1)
    x, _ = synth.outlier_activations(rng, 19, K, max(1, K // 1000), 100.0, dtype=dtype)
    x[3] = 0
    check_fwht_quant(x, 1)


def test_fwht_quant_zero_and_tiny_rows():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 12288)).astype(np.float16)
    x[1] = 0
    x[3] = 0
    x[3, 100] = np.float16(6e-8)                                 # fp16 subnormal
    xq, s, _ = check_fwht_quant(x, 12288)
    assert s[1] == 0 and (xq[1] == 0).all()


def magnitude_rows():
    """fp16 rows of 12288 across the fp16 range: N(0,1) rows scaled by 2^e
    (e = -30 rounds to zero, e = -26 leaves only subnormals and zeros), a constant 65504 row (every
    32-sum of the first Hadamard stage reaches 32 * 65504), rows of random
    +-65504, and rows whose rotated absmax sits near 2 (the matrix-core path
    rescales rows below that)."""
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(12288) * 2.0 ** e for e in (-30, -26, -24, -20, -16, -12, -8, -4, -2, 0, 4, 8, 12)]
    rows.append(np.full(12288, 65504.0))
    rows += [np.where(rng.random(12288) < 0.5, -65504.0, 65504.0) for _ in range(2)]
    base = rng.standard_normal(12288)
    amax = np.abs(base @ oracle.hadamard(12288)).max() / np.sqrt(12288)
    rows += [base * (f / amax) for f in (1.999, 2.0, 2.001)]
    return np.stack(rows).astype(np.float16)


def test_fwht_quant_12288_magnitude_range():
    x = magnitude_rows()
    xq, s, _ = check_fwht_quant(x, 12288)
    assert ((s > 0) == (np.abs(x.astype(np.float32)).max(axis=1) > 0)).all()


@pytest.mark.parametrize("bits", [4, 8])
def test_fwht_quant_12288_both_kernels_agree(bits):
    """Batches of up to 512 rows of 12288 run four waves per row, larger ones
    one wave per row; both must give the same bits.  The magnitude rows (both
    passes of the matrix-core path) lead a batch of 619 rows, checked against
    the oracle, and its first 200 rows are run again as a small batch."""
    rng = np.random.default_rng(12)
    extra, _ = synth.outlier_activations(rng, 600, 12288, 12, 100.0)
    lead = magnitude_rows()
    x = np.concatenate([lead, extra]).astype(np.float16)
    assert x.shape[0] > 512 >= 200
    if bits == 4:
        xq, s, xr = check_fwht_quant(x, 12288, rows=np.r_[0:len(lead), 100, x.shape[0] - 1])
        run = lambda a: spin.spin_fwht_quant(_dev(a), 12288, want_rot=True)
    else:
        run = lambda a: spin.spin_fwht_quant8(_dev(a), 12288, want_rot=True)
        xq, s, xr = (_host(v) for v in run(x))
        c_ref, s_ref = oracle.quantize_rows(xr, 127)
        assert np.array_equal(xq, c_ref) and np.array_equal(s, s_ref)
    xq2, s2, xr2 = (_host(v) for v in run(x[:200]))
    assert np.array_equal(xr2.view(np.uint32), xr[:200].view(np.uint32))
    assert np.array_equal(s2.view(np.uint32), s[:200].view(np.uint32))
    assert np.array_equal(xq2, xq[:200])


def test_fwht_quant_down_config_full_size():
    cfg = synth.down_config()
    rows = np.array([0, 1, 511, 2048, 4095])
    check_fwht_quant(cfg["x"], cfg["had_n"], rows=rows)


# ---------------------------------------------------------------- kv_quant

def check_kv(x, rotate, groups=None):
    X = _dev(x)
    codes, s16, xr = spin.spin_kv_quant(X, rotate, want_rot=True)
    c, s, y = _host(codes), _host(s16), _host(xr)
    c_ref, s_ref = oracle.quantize_kv_groups(y)
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(c, oracle.pack_int4(c_ref))
    T, H, D = x.shape
    flat = x.reshape(T * H, 1, D)
    sel = np.arange(T * H) if groups is None else np.asarray(groups)
    _, _, y_o = oracle.kv_quant(flat[sel], rotate=bool(rotate))
    assert_rows_close(y.reshape(T * H, D)[sel], y_o.reshape(-1, D))
    # rotate-only (Q path) gives the same y
    _, _, xr2 = spin.spin_kv_quant(X, rotate, quantize=False)
    assert np.array_equal(_host(xr2), y)
    return c, s, y


@pytest.mark.parametrize("rotate", [1, 0])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_kv_quant_small(rotate, dtype):
    cfg = synth.kv_config(T=33, H=5)
    check_kv(cfg["k"].astype(dtype), rotate)


def test_kv_quant_full_size_and_qk_invariance():
    cfg = synth.kv_config()
    rng = np.random.default_rng(3)
    groups = rng.choice(4096 * 32, 2048, replace=False)
    _, _, k_rot = check_kv(cfg["k"], 1, groups)
    _, _, q_rot = spin.spin_kv_quant(_dev(cfg["q"]), 1, quantize=False)
    q_rot = _host(q_rot)
    t = np.arange(0, 4096, 8)
    for h in (0, 17, 31):
        lhs = q_rot[t, h] @ k_rot[t, h].T
        rhs = cfg["q"][t, h].astype(np.float32) @ cfg["k"][t, h].astype(np.float32).T
        assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-4
    check_kv(cfg["v"][:512], 0)


# ---------------------------------------------------------------- fold

def check_fold(w, r, r_block, cols=None):
    Wd = _dev(w)
    Rd = None if r is None else _dev(r)
    W_rot, Wq, ws = spin.spin_fold_rotation(Wd, Rd, r_block)
    wr, wq, s = _host(W_rot), _host(Wq), _host(ws)
    c_ref, s_ref = oracle.quantize_rows(wr.T)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(wq, oracle.pack_int4(c_ref))
    sel = np.arange(w.shape[1]) if cols is None else np.asarray(cols)
    ref, _, _ = oracle.fold_rotation(w[:, sel], r, r_block)
    assert_rows_close(wr[:, sel].T, ref.T)
    return wr, wq, s


def test_fold_tiny_haar():
    cfg = synth.tiny_config()
    check_fold(cfg["w"], cfg["r"], 256)


@pytest.mark.parametrize("r_block,K,N", [(256, 256, 40), (12, 192, 17), (96, 384, 33),
                                         (128, 4096, 70), (12288, 12288, 24), (1, 64, 5),
                                         (64, 128, 65)])
def test_fold_hadamard_orders(r_block, K, N):
    rng = np.random.default_rng(r_block + K)
    w = synth.gaussian_weight(rng, K, N)
    check_fold(w, None, r_block)


def test_fold_head_wise_r2():
    rng = np.random.default_rng(21)
    w = synth.gaussian_weight(rng, 4096, 96)
    r2 = synth.haar_orthogonal(rng, 128)
    check_fold(w, r2, 128)


def test_fold_qkv_config_r1_full_size_sampled():
    cfg = synth.qkv_config()
    check_fold(cfg["w"], cfg["r"], 4096, cols=np.arange(0, 6144, 97))


# ---------------------------------------------------------------- gemm

def check_gemm(qx, qw, sx, sw, rows=None, kernel=None):
    Xq, Wq = _dev(oracle.pack_int4(qx)), _dev(oracle.pack_int4(qw))
    Y, acc = spin.spin_w4a4_gemm(Xq, _dev(sx), Wq, _dev(sw), want_acc=True, kernel=kernel)
    Y2, _ = spin.spin_w4a4_gemm(Xq, _dev(sx), Wq, _dev(sw), kernel=kernel)
    y, a = _host(Y), _host(acc)
    assert np.array_equal(y, _host(Y2))
    sel = np.arange(qx.shape[0]) if rows is None else np.asarray(rows)
    a_ref = oracle.gemm_rows(qx, qw, sel)
    assert np.array_equal(a[sel].astype(np.int64), a_ref)
    assert np.array_equal(y[sel], oracle.dequant(a_ref, sx[sel], sw))
    return y, a


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (37, 53, 128), (130, 260, 256), (128, 128, 4096),
                                   (300, 200, 12288), (16, 4096, 4096), (129, 7, 192)])
def test_gemm_ragged(M, N, K):
    rng = np.random.default_rng(M * N + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw)


@pytest.mark.parametrize("M,N,K", [(1, 37, 128), (5, 4096 + 16, 4096), (16, 6144, 4096),
                                   (16, 4096, 12288), (7, 24576, 4096), (16, 100, 384)])
def test_gemm_decode_sizes(M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw)


@pytest.mark.parametrize("M,N,K", [(17, 37, 128), (32, 300, 1280), (33, 4096 + 16, 4096), (48, 6144, 4096),
                                   (64, 256, 256), (64, 4096, 12288), (61, 24576, 4096), (64, 100, 384),
                                   (65, 333, 512), (96, 4096, 4096), (100, 1000, 12288), (128, 4096, 12288)])
def test_gemm_up_to_128_rows(M, N, K):
    """17 to 128 rows run the weight-streaming kernel with up to eight 16-row
    groups sharing each weight load: all rows, against the int64 oracle, with
    the -8 / +7 extremes in the first and last rows."""
    rng = np.random.default_rng(M * 11 + N + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qx[0] = -8
    qx[M - 1] = 7
    qw[0] = -8
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw)


@pytest.mark.parametrize("M", [16, 17, 64, 65, 128, 129])
@pytest.mark.parametrize("N", [16368, 16400])
def test_gemm_dispatch_boundaries(M, N):
    """Either side of every kernel-choice boundary: 16 / 17 and 64 / 65 rows
    (row groups of the weight-streaming kernel), 128 / 129 rows (its end), and
    a column grid just below and just above 4 x 256 workgroups of 16 columns
    (two waves per workgroup instead of eight; past 64 rows, the tiles).  All
    rows against the int64 oracle."""
    K = 1024
    rng = np.random.default_rng(M * 3 + N)
    qx = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw)


@pytest.mark.parametrize("K", [128, 256, 384, 4096])
def test_gemm_qkv_shape_wide_tiles(K):
    """M = 4096, N = 6144 (qkv_proj) runs 256 x 384 tiles: one step (shorter
    than the load pipeline), two, three and the full K = 4096; sampled rows
    from every row block, all columns."""
    rng = np.random.default_rng(K + 5)
    M, N = 4096, 6144
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw, rows=[0, 1, 127, 255, 256, 2047, 3969, 4095])


def test_gemm_extreme_accumulators():
    K = 12288
    qx = np.full((3, K), 7, np.int8)
    qx[1] = -7
    qx[2, ::2] = -8                                              # -8 nibbles are accepted
    qw = np.full((2, K), -7, np.int8)
    qw[1] = 7
    _, a = check_gemm(qx, qw, np.ones(3, np.float32), np.ones(2, np.float32))
    assert a[0, 0] == -49 * K and a[1, 0] == 49 * K


@pytest.mark.parametrize("M", [3, 17])
def test_gemm_largest_k(M):
    """K = SPIN_GEMM_MAX_K = 171136 with every code at +-7: |acc| = 49 K, and the
    kernels' internal 256-scaled sum 49 * 256 * K sits just below 2^31.  M = 3
    takes the decode kernel, M = 17 the tiled one."""
    K = 171136
    qx = np.full((M, K), 7, np.int8)
    qx[1] = -7
    qw = np.full((2, K), 7, np.int8)
    qw[1, K // 2:] = -7
    _, a = check_gemm(qx, qw, np.ones(M, np.float32), np.ones(2, np.float32))
    assert a[0, 0] == 49 * K and a[1, 0] == -49 * K and a[0, 1] == 0


def test_gemm_down_config_shape_sampled():
    rng = np.random.default_rng(22)
    M, N, K = 4096, 4096, 12288
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw, rows=[0, 1, 127, 128, 2047, 4095])


# ---------------------------------------------------------------- end to end

def test_tiny_chain_end_to_end():
    """Tiny workload, both chains: (i) Hadamard on X, W folded with H_256;
    (ii) X rotated by R upstream, W folded with R."""
    cfg = synth.tiny_config()
    x, w, r = cfg["x"], cfg["w"], cfg["r"]
    # (i)
    Xq, xs, _ = spin.spin_fwht_quant(_dev(x), 256)
    _, Wq, ws = spin.spin_fold_rotation(_dev(w), None, 256)
    Y, _ = spin.spin_w4a4_gemm(Xq, xs, Wq, ws)
    pk, s_o, _ = oracle.fwht_quant(x, 256)
    _, wq_o, ws_o = oracle.fold_rotation(w, None, 256)
    y_o, _ = oracle.w4a4_gemm(pk, s_o, wq_o, ws_o)
    assert_y_close(_host(Y), y_o)
    # (ii)
    xr = (x.astype(np.float64) @ r.astype(np.float64)).astype(np.float32)
    Xq, xs, _ = spin.spin_fwht_quant(_dev(xr), 1)
    _, Wq, ws = spin.spin_fold_rotation(_dev(w), _dev(r), 256)
    Y, _ = spin.spin_w4a4_gemm(Xq, xs, Wq, ws)
    pk, s_o, _ = oracle.fwht_quant(xr, 1)
    _, wq_o, ws_o = oracle.fold_rotation(w, r, 256)
    y_o, _ = oracle.w4a4_gemm(pk, s_o, wq_o, ws_o)
    assert_y_close(_host(Y), y_o)


def test_down_chain_end_to_end_sampled():
    cfg = synth.down_config()
    x, w = cfg["x"], cfg["w"]
    Xq, xs, _ = spin.spin_fwht_quant(_dev(x), 12288)
    _, Wq, ws = spin.spin_fold_rotation(_dev(w), None, 12288)
    Y, acc = spin.spin_w4a4_gemm(Xq, xs, Wq, ws, want_acc=True)
    rows = np.array([0, 777, 4095])
    cols = np.arange(0, 4096, 64)
    pk, s_o, _ = oracle.fwht_quant(x[rows], 12288)
    _, wq_o, ws_o = oracle.fold_rotation(w[:, cols], None, 12288)
    a_o = oracle.gemm_rows(oracle.unpack_int4(pk), oracle.unpack_int4(wq_o), np.arange(3))
    y_o = oracle.dequant(a_o, s_o, ws_o)
    fr = code_flips(_host(Xq)[rows], pk, axis=1)
    fc = code_flips(_host(Wq)[cols], wq_o, axis=1)
    assert_y_close(_host(Y)[rows][:, cols], y_o, flip_rows=fr, flip_cols=fc)


@pytest.fixture(scope="module")
def chain_m8192():
    return synth.chain_config()


@pytest.mark.parametrize("layer", ["qkv", "o", "gate_up", "down"])
def test_decoder_chain_m8192_sampled(layer, chain_m8192):
    """The decoder-layer chain at prefill size (M = 8192), each linear at its
    full shape: activation quantization (FWHT-12288 for down, quant-only for
    the others, whose inputs are already in the rotated basis), the weight fold
    (R1 Haar 4096, head-wise R2 Haar 128, H_12288) and the GEMM.  Codes and
    scales bit-exact with the oracle quantizer on the GPU's own rotated values
    for sampled rows, accumulators bit-exact with the oracle's int64 GEMM on
    the GPU's codes, and Y end to end against the oracle chain on sampled rows
    and columns."""
    L = chain_m8192[layer]
    x, w, r, r_block, had_n = L["x"], L["w"], L["r"], L["r_block"], L["had_n"]
    M, N = x.shape[0], w.shape[1]
    rows = np.array([0, 1, 4097, M - 1])
    cols = np.arange(0, N, N // 64)
    Xq, xs, Xr = spin.spin_fwht_quant(_dev(x), had_n, want_rot=True)
    _, Wq, ws = spin.spin_fold_rotation(_dev(w), None if r is None else _dev(r), r_block)
    Y, acc = spin.spin_w4a4_gemm(Xq, xs, Wq, ws, want_acc=True)
    sel = torch.from_numpy(rows).to(DEV)
    xq_s, xs_s, xr_s = _host(Xq[sel]), _host(xs[sel]), _host(Xr[sel])
    y_s, a_s = _host(Y[sel]), _host(acc[sel])
    c_ref, s_ref = oracle.quantize_rows(xr_s)
    assert np.array_equal(xs_s, s_ref) and np.array_equal(xq_s, oracle.pack_int4(c_ref))
    qx = oracle.unpack_int4(xq_s)
    qw = oracle.unpack_int4(_host(Wq))
    a_ref = oracle.gemm_rows(qx, qw, np.arange(len(rows)))
    assert np.array_equal(a_s.astype(np.int64), a_ref)
    assert np.array_equal(y_s, oracle.dequant(a_ref, xs_s, _host(ws)))
    # end to end against the oracle's own chain on sampled rows and columns
    pk, s_o, y_rot = oracle.fwht_quant(x[rows], had_n)
    assert_rows_close(xr_s, y_rot)
    _, wq_o, ws_o = oracle.fold_rotation(w[:, cols], r, r_block)
    a_o = oracle.gemm_rows(oracle.unpack_int4(pk), oracle.unpack_int4(wq_o), np.arange(len(rows)))
    y_o = oracle.dequant(a_o, s_o, ws_o)
    fr = code_flips(xq_s, pk, axis=1)
    fc = code_flips(_host(Wq)[cols], wq_o, axis=1)
    assert_y_close(y_s[:, cols], y_o, flip_rows=fr, flip_cols=fc)


def test_repeat_runs_are_deterministic():
    cfg = synth.down_config(M=256)
    X = _dev(cfg["x"])
    a = [_host(spin.spin_fwht_quant(X, 12288)[0]) for _ in range(3)]
    assert all(np.array_equal(a[0], b) for b in a[1:])


def test_decode_chain_graph_replays_match_eager():
    """A decode-sized chain (quant-only + GEMM, then FWHT-12288 + GEMM, M = 16)
    captured in one HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager results bit for bit."""
    rng = np.random.default_rng(7)
    M = 16

    def codes(r, c):
        q = rng.integers(-7, 8, size=(r, c)).astype(np.int64)
        return _dev(((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8))

    xa = _dev(rng.standard_normal((M, 4096)).astype(np.float16))
    xb = _dev(rng.standard_normal((M, 12288)).astype(np.float16))
    wa, wsa = codes(1024, 4096), _dev(rng.random(1024).astype(np.float32))
    wb, wsb = codes(512, 12288), _dev(rng.random(512).astype(np.float32))
    bufs = {
        "xqa": torch.empty((M, 2048), dtype=torch.uint8, device=DEV),
        "sa": torch.empty((M,), dtype=torch.float32, device=DEV),
        "ya": torch.empty((M, 1024), dtype=torch.float32, device=DEV),
        "xqb": torch.empty((M, 6144), dtype=torch.uint8, device=DEV),
        "sb": torch.empty((M,), dtype=torch.float32, device=DEV),
        "yb": torch.empty((M, 512), dtype=torch.float32, device=DEV),
    }

    def chain():
        spin.spin_fwht_quant(xa, 1, Xq=bufs["xqa"], x_scale=bufs["sa"])
        spin.spin_w4a4_gemm(bufs["xqa"], bufs["sa"], wa, wsa, Y=bufs["ya"])
        spin.spin_fwht_quant(xb, 12288, Xq=bufs["xqb"], x_scale=bufs["sb"])
        spin.spin_w4a4_gemm(bufs["xqb"], bufs["sb"], wb, wsb, Y=bufs["yb"])

    chain()
    eager = {k: _host(v).copy() for k, v in bufs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        chain()
    for rep in range(4):
        for v in bufs.values():
            v.fill_(0x5A if v.dtype == torch.uint8 else -1)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        for k, v in bufs.items():
            assert np.array_equal(_host(v), eager[k]), f"replay {rep}: {k} differs from eager"
    # and the eager quant-only codes are the oracle's (no rotation: exact)
    pk, s_o, _ = oracle.fwht_quant(_host(xa), 1)
    assert np.array_equal(pk, eager["xqa"]) and np.array_equal(s_o, eager["sa"])


# ---------------------------------------------------------------- rotation-choice probe

def test_library_hadamard_matches_oracle():
    from rotation_bit_quantization_amd import probe
    for n in (256, 768, 1024):
        h = _host(probe.library_hadamard(n)).astype(np.float64)
        ref = oracle.hadamard(n) / np.sqrt(np.float64(n))
        assert np.abs(h - ref).max() <= 1e-6 * np.abs(ref).max()


def test_rotation_probe_matches_oracle():
    """Every error the probe reports (no rotation, Hadamard, randomised
    Hadamards diag(s) H, Haar rotations) equals the oracle's for the same float32
    rotation within 1%, and one randomised-Hadamard layer output matches the
    oracle elementwise (codes bit-exact up to near-tie flips)."""
    from rotation_bit_quantization_amd import probe
    cfg = synth.probe_config(T=64, K=256, N=128, draws=3)
    res = probe.rotation_probe(cfg)
    x, w = cfg["x"], cfg["w"]
    K = x.shape[1]
    y_ref = x.astype(np.float64) @ w.astype(np.float64)
    H = (oracle.hadamard(K) / np.sqrt(np.float64(K))).astype(np.float32)

    def run(R):
        _, xq, xs = oracle.fold_rotation(np.ascontiguousarray(x.T), R, K)
        _, wq, ws = oracle.fold_rotation(w, R, K)
        y, _ = oracle.w4a4_gemm(xq, xs, wq, ws)
        return y, xq, wq

    def err(R):
        y = run(R)[0].astype(np.float64)
        return np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)

    assert abs(res["none"] - err(np.eye(K, dtype=np.float32))) <= 1e-2 * res["none"]
    assert abs(res["hadamard"] - err(H)) <= 1e-2 * res["hadamard"]
    for got, s in zip(res["errors"]["randomized_hadamard"], cfg["signs"]):
        assert abs(got - err((s[:, None] * H).astype(np.float32))) <= 1e-2 * got
    for got, r in zip(res["errors"]["haar"], cfg["haar"]):
        assert abs(got - err(r)) <= 1e-2 * got
    # elementwise, one randomised Hadamard
    R = (cfg["signs"][0][:, None] * H).astype(np.float32)
    y_o, xq_o, wq_o = run(R)
    r_dev = _dev(R)
    _, xq, xs = spin.spin_fold_rotation(_dev(np.ascontiguousarray(x.T)), r_dev, K)
    _, wq, ws = spin.spin_fold_rotation(_dev(w), r_dev, K)
    y, _ = spin.spin_w4a4_gemm(xq, xs, wq, ws)
    fr = code_flips(_host(xq), xq_o, axis=1)
    fc = code_flips(_host(wq), wq_o, axis=1)
    assert_y_close(_host(y), y_o, flip_rows=fr, flip_cols=fc)


# ---------------------------------------------------------------- learned R2 (Cayley SGD)

def test_r2_experiment_errors_match_oracle():
    """The errors the R2 experiment measures through libspin (random
    Hadamards and the learned rotation, block 128) equal the oracle's W4A4
    layer error for the same float32 rotations within 1%, and the learned
    rotation's layer matches the oracle elementwise."""
    from rotation_bit_quantization_amd import cayley
    cfg = synth.r2_config(T=128, heads=8, head_dim=128, N=256, draws=3)
    res = cayley.r2_experiment(cfg, iters=8)
    x, w = cfg["x"], cfg["w"]
    ref = x.astype(np.float64) @ w.astype(np.float64)

    def err(R):
        _, xq, xs = oracle.fold_rotation(np.ascontiguousarray(x.T), R, 128)
        _, wq, ws = oracle.fold_rotation(w, R, 128)
        y, _ = oracle.w4a4_gemm(xq, xs, wq, ws)
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    H = oracle.hadamard(128) / np.sqrt(128.0)
    draws = [err((s[:, None] * H).astype(np.float32)) for s in cfg["signs"]]
    assert abs(res["random_hadamard"]["min"] - min(draws)) <= 1e-2 * min(draws)
    assert abs(res["learned"] - err(res["R2"])) <= 1e-2 * res["learned"]
    assert res["orthogonality_error"] < 1e-12
    # elementwise, the learned R2: the device fold + GEMM against the oracle's
    # (codes bit-exact up to near-tie flips, Y within the end-to-end tolerance)
    R = np.ascontiguousarray(res["R2"], dtype=np.float32)
    _, xq_o, xs_o = oracle.fold_rotation(np.ascontiguousarray(x.T), R, 128)
    _, wq_o, ws_o = oracle.fold_rotation(w, R, 128)
    y_o, _ = oracle.w4a4_gemm(xq_o, xs_o, wq_o, ws_o)
    r_dev = _dev(R)
    _, xq, xs = spin.spin_fold_rotation(_dev(np.ascontiguousarray(x.T)), r_dev, 128)
    _, wq, ws = spin.spin_fold_rotation(_dev(w), r_dev, 128)
    y, _ = spin.spin_w4a4_gemm(xq, xs, wq, ws)
    fr = code_flips(_host(xq), xq_o, axis=1)
    fc = code_flips(_host(wq), wq_o, axis=1)
    assert_y_close(_host(y), y_o, flip_rows=fr, flip_cols=fc)


def test_orthogonality_check_matches_oracle():
    """checks.orthogonality_error (R^T R folded on the device) against the
    oracle's float64 value, for every kind of R the harness feeds the fold,
    and it flags a non-orthogonal input."""
    from rotation_bit_quantization_amd import checks
    rng = np.random.default_rng(9)
    rs = [synth.haar_orthogonal(rng, 128), synth.haar_orthogonal(rng, 1024),
          (oracle.hadamard(256) / np.sqrt(256.0)).astype(np.float32)]
    for r in rs:
        got = checks.orthogonality_error(_dev(r))
        ref = oracle.orthogonality_error(r)
        assert got <= ref + r.shape[0] * 2.0 ** -24 * 4
    bad = rs[0].copy()
    bad[3, 5] += 1e-3                                 # R^T R moves by ~2e-4
    got, ref = checks.orthogonality_error(_dev(bad)), oracle.orthogonality_error(bad)
    assert ref > 1e-4 and abs(got - ref) <= 1e-2 * ref
