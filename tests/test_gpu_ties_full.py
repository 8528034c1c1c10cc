"""GPU parity on the quantizers' near-tie windows and at full workload size.

The fast quantizers (quant-only rows, both 12288-wide Hadamard kernels and
kv_quant, 4- and 8-bit) form y / s with a multiply by an approximate
reciprocal and fall back to the exact IEEE quotient when the estimate lies
within a few grid units of a half-integer.  Random data reaches that window
only by chance, so every test here places values on it on purpose: exact
ties (k + 1/2) s, their float32 neighbours and offsets of a few grid units,
over every fp16 scale significand for the KV path.  The codes must equal the
oracle quantizer's on the GPU's own float32 values bit for bit.

The full-size tests compare every row of the down_proj and qkv_proj GEMMs
with the oracle's int64 product, and 64 rows of the 12288-wide rotation
with the oracle's float64 dense product.
"""

import numpy as np
import pytest
import torch

import oracle
from rotation_bit_quantization_amd import spin, synth
from tests.test_gpu_parity import _dev, _host, assert_rows_close, check_fwht_quant, check_gemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spin.load()


def tie_values(s, qmax, grid_bits, rng, n):
    """n float32 values of magnitude below (qmax - 1/4) s on or near the
    quantizer's ties: fl32((k + 1/2) s), up to four float32 ulps either side,
    and (k + 1/2 +- j 2^-grid_bits) s for j = 1..4, with random signs."""
    s64 = float(s)
    vals = []
    for k in range(qmax):
        t = np.float32((k + 0.5) * s64)
        up, dn = t, t
        vals.append(t)
        for _ in range(4):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
            vals += [up, dn]
        for j in range(1, 5):
            vals.append(np.float32((k + 0.5 + j * 2.0 ** -grid_bits) * s64))
            vals.append(np.float32((k + 0.5 - j * 2.0 ** -grid_bits) * s64))
    vals = np.array(vals, np.float32)
    out = vals[rng.integers(0, len(vals), size=n)]
    return (out * rng.choice(np.array([-1.0, 1.0], np.float32), size=n)).astype(np.float32)


def tie_rows(qmax, grid_bits, M, K, seed):
    """Rows of float32 values whose absmax a (element 0) sets s = fl32(a / qmax)
    and whose other values sit on ties of that s; a spans 40 binades with random
    significands."""
    rng = np.random.default_rng(seed)
    x = np.empty((M, K), np.float32)
    for m in range(M):
        a = np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(-20, 20)))
        s = np.divide(a, np.float32(qmax), dtype=np.float32)
        x[m, 1:] = tie_values(s, qmax, grid_bits, rng, K - 1)
        x[m, 0] = a
    return x


@pytest.mark.parametrize("bits", [4, 8])
def test_quant_only_rows_near_ties(bits):
    """had_n = 1 (quant-only rows, the magic-number quantizer with 1/s) on float32
    rows placed on ties: codes and scales bit-exact with the oracle."""
    qmax, gb = (7, 16) if bits == 4 else (127, 14)
    x = tie_rows(qmax, gb, 96, 4096, seed=bits)
    if bits == 4:
        xq, s, xr = (_host(v) for v in spin.spin_fwht_quant(_dev(x), 1, want_rot=True))
        c_ref, s_ref = oracle.quantize_rows(x)
        assert np.array_equal(xr, x)
        assert np.array_equal(s, s_ref)
        assert np.array_equal(xq, oracle.pack_int4(c_ref))
    else:
        xq, s, xr = (_host(v) for v in spin.spin_fwht_quant8(_dev(x), 1, want_rot=True))
        c_ref, s_ref = oracle.quantize_rows(x, 127)
        assert np.array_equal(s, s_ref) and np.array_equal(xq, c_ref)
    # the rows do reach the ties: a share of the quotients are exact half-integers
    q = np.divide(x[:, 1:], s_ref[:, None], dtype=np.float32)
    assert np.mean(np.abs(q - np.floor(q)) == 0.5) > 0.01


def kv_tie_groups(qmax, grid_bits, seed):
    """[T, 1, 128] float32 vectors whose absmax sets an fp16 scale covering every
    fp16 significand (1024 of them) at three binades and random others, the
    remaining 127 values of each vector on that scale's ties."""
    rng = np.random.default_rng(seed)
    amax = []
    for e in (-13, 0, 12):
        amax += [qmax * (1.0 + m / 1024.0) * 2.0 ** e for m in range(1024)]
    amax += list(qmax * rng.uniform(1.0, 2.0, size=512) * 2.0 ** rng.integers(-13, 15, size=512))
    T = len(amax)
    x = np.empty((T, 1, 128), np.float32)
    for t, a in enumerate(amax):
        a32 = np.float32(a)
        s16 = np.divide(a32, np.float32(qmax), dtype=np.float32).astype(np.float16).astype(np.float32)
        x[t, 0, 1:] = tie_values(s16, qmax, grid_bits, rng, 127)
        x[t, 0, 0] = a32
    return x


@pytest.mark.parametrize("bits", [4, 8])
def test_kv_quant_near_ties_every_fp16_scale(bits):
    """spin_kv_quant(8) with rotate = 0 (the V path, values as given) on float32
    vectors placed on the ties of every fp16 scale significand, where 1/s comes
    from v_rcp_f32: scales and codes bit-exact with the oracle."""
    qmax, gb = (7, 16) if bits == 4 else (127, 14)
    x = kv_tie_groups(qmax, gb, seed=30 + bits)
    run = spin.spin_kv_quant if bits == 4 else spin.spin_kv_quant8
    codes, s16, xr = (_host(v) for v in run(_dev(x), 0, want_rot=True))
    assert np.array_equal(xr, x)
    c_ref, s_ref = oracle.quantize_kv_groups(x, qmax)
    assert np.array_equal(s16.view(np.uint16), s_ref.view(np.uint16))
    if bits == 4:
        assert np.array_equal(codes, oracle.pack_int4(c_ref))
    else:
        assert np.array_equal(codes, c_ref)
    sf = s_ref.astype(np.float32)
    q = np.divide(x[..., 1:], sf[..., None], dtype=np.float32)
    assert np.mean(np.abs(q - np.floor(q)) == 0.5) > 0.01


@pytest.mark.parametrize("bits", [4, 8])
def test_kv_quant_scale_overflow_and_infinite_absmax(bits):
    """float32 KV vectors whose scale overflows fp16 (finite values up to 1e37,
    rotated and not) and vectors holding +inf or -inf among finite values
    (V path): the scale is the fp16 infinity and every finite value's code is 0,
    as for the oracle (codes of infinite values are left unspecified)."""
    qmax = 7 if bits == 4 else 127
    rng = np.random.default_rng(40 + bits)
    x = rng.standard_normal((8, 2, 128)).astype(np.float32)
    x[0, 0, :4] = [1e37, -1e37, 5e36, 1e37]
    x[1, 1, 7] = -3e38
    x[2, 0, 5] = np.inf
    x[3, 1, 0] = -np.inf
    run = spin.spin_kv_quant if bits == 4 else spin.spin_kv_quant8
    unpack = oracle.unpack_int4 if bits == 4 else (lambda c: c)
    for rotate in (0, 1):
        xin = x.copy() if rotate == 0 else x[:2].copy()
        codes, s16, xr = (_host(v) for v in run(_dev(xin), rotate, want_rot=True))
        c_ref, s_ref = oracle.quantize_kv_groups(xr, qmax)
        assert np.array_equal(s16.view(np.uint16), s_ref.view(np.uint16))
        finite = np.isfinite(xr)
        assert np.array_equal(unpack(codes)[finite], c_ref[finite])
        assert (s16.view(np.uint16)[0, 0] & 0x7FFF) == 0x7C00          # fp16 infinity
        if rotate == 0:
            assert (s16.view(np.uint16)[2, 0] & 0x7FFF) == 0x7C00
            assert (unpack(codes)[2, 0][finite[2, 0]] == 0).all()


def hadamard_tie_rows(qmax, M, seed):
    """fp16 rows x = a h_i + sum_t b_t h_{j_t} over columns h of the unnormalised
    H_12288: the rotation x . H / sqrt(n) maps them to sqrt(n) (a e_i + sum b_t
    e_j_t), so with a = 2 qmax and b_t = +-(2 k_t + 1) the absmax sets
    s = sqrt(n) a / qmax and every other non-zero output sits on the tie
    k_t + 1/2 up to float32 rounding.  All entries are small integers (exact
    in fp16) and every partial sum of the transform is exact."""
    rng = np.random.default_rng(seed)
    h12 = oracle.paley12().astype(np.int32)
    h1024 = oracle.sylvester(1024).astype(np.int32)

    def column(c):          # column (a, b) of H12 (x) H1024, c = 1024 a + b
        return np.kron(h12[:, c // 1024], h1024[:, c % 1024])

    x = np.zeros((M, 12288), np.int32)
    for m in range(M):
        cols = rng.choice(12288, size=4, replace=False)
        x[m] += 2 * qmax * column(cols[0]) * (1 if m % 2 else -1)
        for c in cols[1:]:
            b = 2 * int(rng.integers(0, qmax)) + 1
            x[m] += b * column(c) * int(rng.choice([-1, 1]))
    return x.astype(np.float16)


@pytest.mark.parametrize("bits", [4, 8])
def test_fwht_quant_12288_ties_both_kernels(bits):
    """Rows of 12288 whose rotated values sit on the quantizer's ties, through
    the one-wave kernel (a batch of 600 rows) and the four-waves-per-row kernel
    (its first 200 rows again): codes and scales bit-exact with the oracle on
    the GPU's float32 values, and the two kernels bit-identical."""
    qmax = 7 if bits == 4 else 127
    x = hadamard_tie_rows(qmax, 600, seed=50 + bits)
    run = (lambda a: spin.spin_fwht_quant(_dev(a), 12288, want_rot=True)) if bits == 4 else \
        (lambda a: spin.spin_fwht_quant8(_dev(a), 12288, want_rot=True))
    xq, s, xr = (_host(v) for v in run(x))
    c_ref, s_ref = oracle.quantize_rows(xr, qmax)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(xq, oracle.pack_int4(c_ref) if bits == 4 else c_ref)
    q = np.abs(np.divide(xr, s_ref[:, None], dtype=np.float32))
    ties = q[(q != 0) & (q < qmax - 0.25)]
    assert len(ties) == 3 * x.shape[0]
    assert np.all(np.abs(ties - np.floor(ties) - 0.5) < 1e-4)
    sel = np.arange(0, 600, 40)
    _, _, y_o = oracle.fwht_quant(x[sel], 12288)
    assert_rows_close(xr[sel], y_o)
    xq2, s2, xr2 = (_host(v) for v in run(x[:200]))
    assert np.array_equal(xr2.view(np.uint32), xr[:200].view(np.uint32))
    assert np.array_equal(s2, s[:200]) and np.array_equal(xq2, xq[:200])


# ---------------------------------------------------------------- full size

def test_fwht_quant_down_config_64_rows_dense():
    """The down_proj workload (4096 x 12288 fp16): codes and scales of every row
    against the oracle quantizer on the GPU's values, and the rotation of 64
    rows spread over the batch against the oracle's float64 dense product."""
    cfg = synth.down_config()
    rows = np.linspace(0, 4095, 64).astype(np.int64)
    check_fwht_quant(cfg["x"], cfg["had_n"], rows=rows)


@pytest.mark.parametrize("shape", [(4096, 4096, 12288), (4096, 6144, 4096)])
def test_gemm_full_size_every_row(shape):
    """down_proj (4096 x 4096 x 12288) and qkv_proj (4096 x 6144 x 4096): the
    int32 accumulators and Y of every row and column against the oracle."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    qx = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sx = rng.random(M).astype(np.float32)
    sw = (rng.random(N) * 0.01).astype(np.float32)
    check_gemm(qx, qw, sx, sw)
