"""Compile the oracle's C routine (test infrastructure; gcc + OpenMP, no HIP).

    python -m oracle.build      # writes oracle/liboracle_gemm.so
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_int64.c")
LIB = os.path.join(HERE, "liboracle_gemm.so")


def build(force: bool = True) -> str:
    """Compile gemm_int64.c into liboracle_gemm.so and return its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(HERE, "liboracle_gemm_san.so")


def build_sanitized() -> str:
    """The same routine built with AddressSanitizer and UndefinedBehaviorSanitizer
    (no recovery) into liboracle_gemm_san.so; a process loading it preloads
    gcc's libasan (see sanitizer_preload)."""
    tmp = SAN_LIB + ".tmp"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_preload() -> str:
    """LD_PRELOAD value for a process that loads liboracle_gemm_san.so."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True, check=True)
        libs.append(out.stdout.strip())
    return ":".join(libs)


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
