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
    for name in ("spin_probe_mfma", "spin_probe_read"):
        assert hasattr(probe, name)
    NULL, BAD, MIS = 1, 2, 3
    assert probe.spin_probe_mfma(0, 1, 1, None, A, None) == NULL
    assert probe.spin_probe_mfma(2, 1, 1, A, A, None) == BAD
    assert probe.spin_probe_mfma(0, 0, 1, A, A, None) == BAD
    assert probe.spin_probe_mfma(1, 1, 0, A, A, None) == BAD
    assert probe.spin_probe_mfma(0, 1, 1, U, A, None) == MIS
    assert probe.spin_probe_read(None, 16, 1, A, None) == NULL
    assert probe.spin_probe_read(A, 0, 1, A, None) == BAD
    assert probe.spin_probe_read(A, 24, 1, A, None) == BAD
    assert probe.spin_probe_read(A, 16, 0, A, None) == BAD
    assert probe.spin_probe_read(U, 16, 1, A, None) == MIS
