"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* libspin's host side (abi.cpp: every entry point's argument validation and
  dispatch) built with both sanitizers, no recovery, linked with the same GPU
  code objects; the whole C-ABI validation suite (tests/test_abi_cpu.py) runs
  against it in a child process with the sanitizer runtime preloaded.
* The oracle's C GEMM (gemm_int64.c, OpenMP) built the same way with gcc and
  run on ragged shapes, all rows and selected rows, against its float64 BLAS
  route.

A sanitizer report ends the child with a non-zero status and is printed here.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(cmd, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_abi_validation_under_host_sanitizers():
    from rotation_bit_quantization_amd import build
    if not os.path.exists(os.path.join(ROOT, "rotation_bit_quantization_amd", "libspin.so")):
        pytest.skip("libspin.so not built")
    try:
        lib = build.build_host_sanitized()
        rt = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(f"host sanitizer build unavailable: {e}")
    out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                os.path.join("tests", "test_abi_cpu.py")],
               {"LD_PRELOAD": rt, "SPIN_LIBRARY": lib})
    assert " passed" in out and " failed" not in out


ORACLE_SCRIPT = r"""
import numpy as np
import oracle
from oracle import gemm
rng = np.random.default_rng(5)
for M, N, K in [(1, 1, 1), (3, 5, 7), (37, 53, 130), (64, 33, 1024)]:
    qx = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    ref = gemm.gemm_int_codes_blas(qx, qw)
    assert np.array_equal(gemm.gemm_int_codes(qx, qw), ref)
    rows = np.unique(rng.integers(0, M, size=min(M, 5)))
    assert np.array_equal(gemm.gemm_rows(qx, qw, rows), ref[rows])
print("oracle gemm ok", gemm.num_threads())
"""


def test_oracle_gemm_under_sanitizers():
    from oracle import build
    try:
        lib = build.build_sanitized()
        pre = build.sanitizer_preload()
    except (subprocess.CalledProcessError, OSError) as e:
        pytest.skip(f"gcc sanitizer build unavailable: {e}")
    out = _run([sys.executable, "-c", ORACLE_SCRIPT], {"LD_PRELOAD": pre, "ORACLE_GEMM_LIBRARY": lib})
    assert "oracle gemm ok" in out
