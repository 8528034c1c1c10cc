"""libspin C ABI checks that need no GPU: the library loads, exports every
symbol include/libspin.h declares, and every validation error is returned
before any device call (fake, never-dereferenced pointers are used)."""

import ctypes
import os
import re

import pytest

from rotation_bit_quantization_amd import spin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libspin.h")

A = 4096          # a fake 16-byte-aligned device address (never dereferenced)
U = 4097          # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(spin.library_path()):
        pytest.skip("libspin.so not built (python -m rotation_bit_quantization_amd.build)")
    return spin.load()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:spin_status|const char\*|int)\s+(spin_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(spin.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for s in range(6):
        assert spin.spin_status_string(s).startswith("SPIN_")
    assert "unknown" in spin.spin_status_string(99)
    assert lib.spin_version() >= 100


def test_fwht_quant_validation(lib):
    f = lib.spin_fwht_quant
    ok = dict(X=A, dt=spin.SPIN_F16, M=4, K=256, n=256, Xq=A, s=A, r=None, st=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["X"], a["dt"], a["M"], a["K"], a["n"], a["Xq"], a["s"], a["r"], a["st"])

    assert call(X=None) == spin.SPIN_ERR_NULL
    assert call(Xq=None) == spin.SPIN_ERR_NULL
    assert call(s=None) == spin.SPIN_ERR_NULL
    assert call(dt=7) == spin.SPIN_ERR_UNSUPPORTED
    for bad_n in (0, 3, 24576, 32768, 36):
        assert call(n=bad_n) == spin.SPIN_ERR_UNSUPPORTED
    assert call(M=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(K=0) == spin.SPIN_ERR_BAD_SHAPE
    assert call(K=48, n=1) == spin.SPIN_ERR_BAD_SHAPE          # K % 32
    assert call(K=512 + 32, n=256) == spin.SPIN_ERR_BAD_SHAPE   # K % had_n
    assert call(K=65536, n=1) == spin.SPIN_ERR_BAD_SHAPE        # above SPIN_FWHT_MAX_K
    assert call(M=1 << 24) == spin.SPIN_ERR_BAD_SHAPE           # above SPIN_FWHT_MAX_M: one launch's rows
    assert call(M=(1 << 31) - 1, K=32, n=32) == spin.SPIN_ERR_BAD_SHAPE
    assert call(X=U) == spin.SPIN_ERR_MISALIGNED
    assert call(r=U) == spin.SPIN_ERR_MISALIGNED
    assert call(M=0) == spin.SPIN_OK                             # empty: nothing enqueued


def test_gemm_validation(lib):
    f = lib.spin_w4a4_gemm

    def call(Xq=A, sx=A, Wq=A, sw=A, M=16, N=16, K=128, Y=A, acc=None):
        return f(Xq, sx, Wq, sw, M, N, K, Y, acc, None)

    assert call(Xq=None) == spin.SPIN_ERR_NULL
    assert call(Y=None) == spin.SPIN_ERR_NULL
    assert call(K=96) == spin.SPIN_ERR_BAD_SHAPE
    assert call(K=0) == spin.SPIN_ERR_BAD_SHAPE
    assert call(K=171136 + 64) == spin.SPIN_ERR_BAD_SHAPE
    assert call(M=-3) == spin.SPIN_ERR_BAD_SHAPE
    assert call(acc=U) == spin.SPIN_ERR_MISALIGNED
    assert call(sw=U) == spin.SPIN_ERR_MISALIGNED
    assert call(M=0) == spin.SPIN_OK
    assert call(N=0) == spin.SPIN_OK


def test_kv_validation(lib):
    f = lib.spin_kv_quant

    def call(X=A, dt=spin.SPIN_F16, T=4, H=2, D=128, rot=1, c=A, s=A, r=None):
        return f(X, dt, T, H, D, rot, c, s, r, None)

    assert call(X=None) == spin.SPIN_ERR_NULL
    assert call(c=None) == spin.SPIN_ERR_NULL                    # codes / scale must pair
    assert call(c=None, s=None, r=None) == spin.SPIN_ERR_NULL    # nothing to write
    assert call(rot=2) == spin.SPIN_ERR_UNSUPPORTED
    assert call(D=64) == spin.SPIN_ERR_BAD_SHAPE
    assert call(T=-1) == spin.SPIN_ERR_BAD_SHAPE
    # SPIN_KV_MAX_VECTORS = (2^24 - 1) * 32: 32 past it, one past it, far past it
    assert call(T=1 << 24, H=32) == spin.SPIN_ERR_BAD_SHAPE
    assert call(T=((1 << 24) - 1) * 32 + 1, H=1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(T=1 << 30, H=1 << 4) == spin.SPIN_ERR_BAD_SHAPE
    assert call(s=U) == spin.SPIN_ERR_MISALIGNED
    assert call(T=0) == spin.SPIN_OK


def test_fold_validation(lib):
    f = lib.spin_fold_rotation

    def call(W=A, K=256, N=64, R=A, r=256, Wr=A, Wq=A, ws=A):
        return f(W, K, N, R, r, Wr, Wq, ws, None)

    assert call(W=None) == spin.SPIN_ERR_NULL
    assert call(Wr=None) == spin.SPIN_ERR_NULL
    assert call(r=0) == spin.SPIN_ERR_BAD_SHAPE
    assert call(R=None, r=48) == spin.SPIN_ERR_BAD_SHAPE          # 256 % 48 -> shape after order check
    assert call(R=None, r=5) == spin.SPIN_ERR_UNSUPPORTED
    assert call(K=96, r=32) == spin.SPIN_ERR_BAD_SHAPE            # K % 64
    assert call(K=256, r=96) == spin.SPIN_ERR_BAD_SHAPE           # K % r_block
    assert call(R=U) == spin.SPIN_ERR_MISALIGNED
    assert call(N=0) == spin.SPIN_OK


def test_fwht_quant8_validation(lib):
    f = lib.spin_fwht_quant8

    def call(X=A, dt=spin.SPIN_F16, M=4, K=256, n=256, Xq=A, s=A, r=None):
        return f(X, dt, M, K, n, Xq, s, r, None)

    assert call(Xq=None) == spin.SPIN_ERR_NULL
    assert call(n=3) == spin.SPIN_ERR_UNSUPPORTED
    assert call(K=48, n=1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(Xq=U) == spin.SPIN_ERR_MISALIGNED
    assert call(M=0) == spin.SPIN_OK


def test_w4a8_gemm_validation(lib):
    f = lib.spin_w4a8_gemm

    def call(Xq=A, sx=A, Wq=A, sw=A, M=16, N=16, K=256, Y=A, acc=None):
        return f(Xq, sx, Wq, sw, M, N, K, Y, acc, None)

    assert call(Xq=None) == spin.SPIN_ERR_NULL
    assert call(sw=None) == spin.SPIN_ERR_NULL
    assert call(K=64) == spin.SPIN_ERR_BAD_SHAPE                  # K % 128
    assert call(K=150912 + 128) == spin.SPIN_ERR_BAD_SHAPE        # above SPIN_GEMM8_MAX_K
    assert call(N=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(Xq=U) == spin.SPIN_ERR_MISALIGNED
    assert call(M=0) == spin.SPIN_OK


def test_kv_quant8_validation(lib):
    f = lib.spin_kv_quant8

    def call(X=A, dt=spin.SPIN_F16, T=4, H=2, D=128, rot=1, c=A, s=A, r=None):
        return f(X, dt, T, H, D, rot, c, s, r, None)

    assert call(s=None) == spin.SPIN_ERR_NULL
    assert call(D=256) == spin.SPIN_ERR_BAD_SHAPE
    assert call(dt=3) == spin.SPIN_ERR_UNSUPPORTED
    assert call(c=U) == spin.SPIN_ERR_MISALIGNED
    assert call(H=0) == spin.SPIN_OK


def test_gemm_ex_validation(lib):
    f = lib.spin_w4a4_gemm_ex

    def call(M=4, N=4, K=8192, kernel=spin.SPIN_GEMM_FP6, y=A):
        return f(A, A, A, A, M, N, K, y, None, kernel, None)

    assert call(kernel=4) == spin.SPIN_ERR_UNSUPPORTED
    assert call(kernel=-1) == spin.SPIN_ERR_UNSUPPORTED
    for k in (spin.SPIN_GEMM_FP6, spin.SPIN_GEMM_FP6_SPLITK):
        assert call(K=128, kernel=k) == spin.SPIN_ERR_BAD_SHAPE         # below the FP6 pipeline's two steps
        assert call(K=8192 + 64, kernel=k) == spin.SPIN_ERR_BAD_SHAPE   # not a multiple of 128
        assert call(K=65536 + 128, kernel=k) == spin.SPIN_ERR_BAD_SHAPE # beyond exact float32 accumulation
        assert call(K=256, M=0, kernel=k) == spin.SPIN_OK
    assert call(K=65536 + 128, kernel=spin.SPIN_GEMM_INT8, y=None) == spin.SPIN_ERR_NULL
    assert call(K=65536 + 128, kernel=spin.SPIN_GEMM_INT8, M=0) == spin.SPIN_OK
    assert call(K=256, M=0) == spin.SPIN_OK
    assert call(y=None) == spin.SPIN_ERR_NULL
    assert call(y=U) == spin.SPIN_ERR_MISALIGNED


def test_gemm_fp6_k_range_is_the_float32_limit():
    """SPIN_GEMM_FP6_MAX_K: the float32 accumulator of products u_a * u_b <= 225
    (u = q + 8 in [0, 15]) is exact while 225 K stays below 2^24 (K < 74566);
    the library stops at the power of two below that."""
    text = open(HEADER).read()
    kmax = int(re.search(r"#define SPIN_GEMM_FP6_MAX_K (\d+)", text).group(1))
    kmin = int(re.search(r"#define SPIN_GEMM_FP6_MIN_K (\d+)", text).group(1))
    assert kmax % 128 == 0 and 225 * kmax < 2 ** 24
    assert kmin == 256


def test_fwht_quant_gemm_validation(lib):
    f = lib.spin_fwht_quant_gemm

    def call(X=A, dt=spin.SPIN_F16, M=4, K=12288, had=12288, w=A, ws_=A, N=8, xq=A, xs=A, y=A, acc=None,
             work=A):
        return f(X, dt, M, K, had, w, ws_, N, xq, xs, y, acc, work, None)

    for name in ("X", "w", "ws_", "xq", "xs", "y", "work"):
        assert call(**{name: None}) == spin.SPIN_ERR_NULL, name
    assert call(dt=spin.SPIN_F32) == spin.SPIN_ERR_UNSUPPORTED
    assert call(had=4096) == spin.SPIN_ERR_UNSUPPORTED
    assert call(K=4096) == spin.SPIN_ERR_BAD_SHAPE
    assert call(M=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(M=1 << 24) == spin.SPIN_ERR_BAD_SHAPE
    assert call(N=-1) == spin.SPIN_ERR_BAD_SHAPE
    for name in ("X", "w", "ws_", "xq", "xs", "y", "acc", "work"):
        assert call(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    assert call(M=0) == spin.SPIN_OK


def test_fwht_quant_gemm_noalloc_validation(lib):
    """The allocation-free variant validates like the workspace one, before it
    touches its per-device flags (so no GPU is needed for these)."""
    f = lib.spin_fwht_quant_gemm_noalloc

    def call(X=A, dt=spin.SPIN_F16, M=4, K=12288, had=12288, w=A, ws_=A, N=8, xq=A, xs=A, y=A, acc=None):
        return f(X, dt, M, K, had, w, ws_, N, xq, xs, y, acc, None)

    for name in ("X", "w", "ws_", "xq", "xs", "y"):
        assert call(**{name: None}) == spin.SPIN_ERR_NULL, name
    assert call(dt=spin.SPIN_F32) == spin.SPIN_ERR_UNSUPPORTED
    assert call(had=4096) == spin.SPIN_ERR_UNSUPPORTED
    assert call(K=4096) == spin.SPIN_ERR_BAD_SHAPE
    assert call(M=-1) == spin.SPIN_ERR_BAD_SHAPE
    for name in ("X", "w", "ws_", "xq", "xs", "y", "acc"):
        assert call(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    assert call(M=0) == spin.SPIN_OK


def test_f6_pair_validation(lib):
    f = lib.spin_fwht_quant_f6

    def q6(X=A, dt=spin.SPIN_F16, M=4, K=12288, had=12288, xf=A, xsum=A, xs=A):
        return f(X, dt, M, K, had, xf, xsum, xs, None)

    for name in ("X", "xf", "xsum", "xs"):
        assert q6(**{name: None}) == spin.SPIN_ERR_NULL, name
        assert q6(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    assert q6(dt=spin.SPIN_F32) == spin.SPIN_ERR_UNSUPPORTED
    assert q6(had=4096) == spin.SPIN_ERR_UNSUPPORTED
    assert q6(K=4096) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(M=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(M=1 << 24) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(M=0) == spin.SPIN_OK
    # had_n = 1 (quant only): fp16 / fp32, K % 128 == 0, 256 <= K <= SPIN_FWHT_F6_QUANT_MAX_K
    assert q6(had=2, K=4096) == spin.SPIN_ERR_UNSUPPORTED
    assert q6(had=1, K=4096, dt=7) == spin.SPIN_ERR_UNSUPPORTED
    assert q6(had=1, K=4096 + 64) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(had=1, K=128) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(had=1, K=16384 + 128) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(had=1, K=4096, M=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert q6(had=1, K=4096, X=U) == spin.SPIN_ERR_MISALIGNED
    assert q6(had=1, K=4096, dt=spin.SPIN_F32, M=0) == spin.SPIN_OK

    g = lib.spin_w4a4_gemm_f6

    def g6(xf=A, xsum=A, xs=A, w=A, ws_=A, M=4, N=4, K=12288, y=A, acc=None):
        return g(xf, xsum, xs, w, ws_, M, N, K, y, acc, None)

    for name in ("xf", "xsum", "xs", "w", "ws_", "y"):
        assert g6(**{name: None}) == spin.SPIN_ERR_NULL, name
    for name in ("xf", "xsum", "xs", "w", "ws_", "y", "acc"):
        assert g6(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    assert g6(K=128) == spin.SPIN_ERR_BAD_SHAPE
    assert g6(K=8192 + 64) == spin.SPIN_ERR_BAD_SHAPE
    assert g6(K=65536 + 128) == spin.SPIN_ERR_BAD_SHAPE
    assert g6(M=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert g6(M=0) == spin.SPIN_OK and g6(N=0) == spin.SPIN_OK


def test_codes_f6_validation(lib):
    f = lib.spin_codes_f6

    def w6(w=A, N=4, K=12288, wf=A, wsum=A):
        return f(w, N, K, wf, wsum, None)

    for name in ("w", "wf", "wsum"):
        assert w6(**{name: None}) == spin.SPIN_ERR_NULL, name
        assert w6(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    assert w6(K=0) == spin.SPIN_ERR_BAD_SHAPE
    assert w6(K=96) == spin.SPIN_ERR_BAD_SHAPE
    assert w6(K=171136 + 64) == spin.SPIN_ERR_BAD_SHAPE
    assert w6(N=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert w6(N=0) == spin.SPIN_OK

    g = lib.spin_w4a4_gemm_f6f6

    def g66(xf=A, xsum=A, xs=A, wf=A, wsum=A, ws_=A, M=4, N=4, K=12288, y=A, acc=None):
        return g(xf, xsum, xs, wf, wsum, ws_, M, N, K, y, acc, None)

    for name in ("xf", "xsum", "xs", "wf", "wsum", "ws_", "y"):
        assert g66(**{name: None}) == spin.SPIN_ERR_NULL, name
    for name in ("xf", "xsum", "xs", "wf", "wsum", "ws_", "y", "acc"):
        assert g66(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    assert g66(K=128) == spin.SPIN_ERR_BAD_SHAPE
    assert g66(K=8192 + 64) == spin.SPIN_ERR_BAD_SHAPE
    assert g66(K=65536 + 128) == spin.SPIN_ERR_BAD_SHAPE
    assert g66(N=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert g66(M=0) == spin.SPIN_OK and g66(N=0) == spin.SPIN_OK


def test_kv_qkv_validation(lib):
    f = lib.spin_kv_qkv

    def call(Q=A, K=A, V=A, dt=spin.SPIN_F16, T=4, Hq=4, Hkv=2, D=128, bits=4, qr=A, kc=A, ks=A, kr=None,
             vc=A, vs=A):
        return f(Q, K, V, dt, T, Hq, Hkv, D, bits, qr, kc, ks, kr, vc, vs, None)

    for name in ("K", "V", "kc", "ks", "vc", "vs"):
        assert call(**{name: None}) == spin.SPIN_ERR_NULL, name
    assert call(qr=None) == spin.SPIN_ERR_NULL                  # Q without Q_rot
    assert call(Q=None) == spin.SPIN_ERR_NULL                   # Q_rot without Q
    assert call(dt=2) == spin.SPIN_ERR_UNSUPPORTED
    assert call(bits=6) == spin.SPIN_ERR_UNSUPPORTED
    assert call(D=64) == spin.SPIN_ERR_BAD_SHAPE
    assert call(T=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(Hkv=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(Hq=-1) == spin.SPIN_ERR_BAD_SHAPE
    assert call(T=1 << 30, Hkv=32) == spin.SPIN_ERR_BAD_SHAPE   # 2^35 vectors
    assert call(T=1 << 30, Hkv=1, Hq=32) == spin.SPIN_ERR_BAD_SHAPE
    # the one launch holds 2 ceil(T Hkv / 32) + ceil(T Hq / 32) < 2^24 workgroups
    assert call(T=1 << 20, Hkv=128, Hq=256) == spin.SPIN_ERR_BAD_SHAPE      # exactly 2^24
    assert call(T=1 << 23, Hkv=32, Q=None, qr=None) == spin.SPIN_ERR_BAD_SHAPE
    for name in ("Q", "K", "V", "qr", "kc", "ks", "kr", "vc", "vs"):
        assert call(**{name: U}) == spin.SPIN_ERR_MISALIGNED, name
    # Hq is ignored without Q; empty problems enqueue nothing
    assert call(Q=None, qr=None, Hq=-1, T=0) == spin.SPIN_OK
    assert call(T=0) == spin.SPIN_OK
    assert call(Q=None, qr=None, Hkv=0) == spin.SPIN_OK
    assert call(Hq=0, Hkv=0) == spin.SPIN_OK


def test_gemm8_bound_is_the_int32_limit():
    """SPIN_GEMM8_MAX_K: the largest multiple of 128 with 127 * 7 * 16 * K < 2^31."""
    k = 150912
    assert k % 128 == 0 and 127 * 7 * 16 * k < 2 ** 31 and 127 * 7 * 16 * (k + 128) >= 2 ** 31
    assert "#define SPIN_GEMM8_MAX_K 150912" in open(HEADER).read()


# ---------------------------------------------------------------- libspin_probe

PROBE_HEADER = os.path.join(ROOT, "include", "spin_probe.h")


@pytest.fixture(scope="module")
def probe():
    from rotation_bit_quantization_amd import machine
    if not os.path.exists(machine.library_path()):
        pytest.skip("libspin_probe.so not built (python -m rotation_bit_quantization_amd.build)")
    return machine.load()


def test_probe_header_declares_the_binding_symbols():
    from rotation_bit_quantization_amd import machine
    text = open(PROBE_HEADER).read()
    declared = sorted(set(re.findall(r"^\s*spin_status\s+(spin_\w+)\s*\(", text, re.M)))
    assert declared == sorted(machine.EXPORTED_SYMBOLS)


def test_probe_symbols_and_validation(probe):
    for name in ("spin_probe_mfma", "spin_probe_read", "spin_probe_lds"):
        assert hasattr(probe, name)
    NULL, BAD, MIS = 1, 2, 3
    assert probe.spin_probe_mfma(0, 1, 1, None, A, None) == NULL
    assert probe.spin_probe_mfma(3, 1, 1, A, A, None) == BAD
    assert probe.spin_probe_mfma(-1, 1, 1, A, A, None) == BAD
    assert probe.spin_probe_mfma(0, 0, 1, A, A, None) == BAD
    assert probe.spin_probe_mfma(1, 1, 0, A, A, None) == BAD
    assert probe.spin_probe_mfma(0, 1, 1, U, A, None) == MIS
    assert probe.spin_probe_read(None, 16, 1, A, None) == NULL
    assert probe.spin_probe_read(A, 0, 1, A, None) == BAD
    assert probe.spin_probe_read(A, 24, 1, A, None) == BAD
    assert probe.spin_probe_read(A, 16, 0, A, None) == BAD
    assert probe.spin_probe_read(U, 16, 1, A, None) == MIS
    assert probe.spin_probe_lds(0, 1, 1, None, A, None) == NULL
    assert probe.spin_probe_lds(0, 1, 1, A, None, None) == NULL
    assert probe.spin_probe_lds(3, 1, 1, A, A, None) == BAD
    assert probe.spin_probe_lds(-1, 1, 1, A, A, None) == BAD
    assert probe.spin_probe_lds(0, 0, 1, A, A, None) == BAD
    assert probe.spin_probe_lds(2, 1, 0, A, A, None) == BAD
    assert probe.spin_probe_lds(1, 1, 1, U, A, None) == MIS
