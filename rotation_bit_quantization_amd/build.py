"""Build libspin.so (and the benchmark's machine probes, libspin_probe.so)
in-tree with hipcc for gfx950.

    python -m rotation_bit_quantization_amd.build

Each source is compiled to an object in parallel, then linked into
``rotation_bit_quantization_amd/libspin.so``; ``machine_probe.hip`` goes into
``libspin_probe.so`` on its own.  Every HIP source is compiled with the
packed-fp32 VALU forms disabled.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspin.so")
SOURCES = ["abi.cpp", "fwht_quant.hip", "kv_quant.hip", "fold.hip", "w4a4_gemm.hip", "w4a4_gemm_fp6.hip",
           "fwht_quant_gemm.hip", "w4a8_gemm.hip", "quant_f6.hip"]
PROBE_LIB = os.path.join(PKG, "libspin_probe.so")
PROBE_SOURCES = ["machine_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libspin needs ROCm to build")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


HOSTSAN_LIB = os.path.join(OBJ, "libspin_hostsan.so")


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it also holds
    the UndefinedBehaviorSanitizer handlers); a process loading the
    host-sanitized library preloads it."""
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm), reverse=True) if os.path.isdir(llvm) else []:
        rt = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(rt):
            return rt
    raise RuntimeError("clang AddressSanitizer runtime not found")


def build_host_sanitized() -> str:
    """Link a second libspin, libspin_hostsan.so under _build/, whose host
    code (abi.cpp: argument validation, dispatch, scratch and occupancy
    caches) is built with AddressSanitizer and UndefinedBehaviorSanitizer
    (no recovery); the GPU code objects are the ones build() compiled.  Each
    sanitizer flag applies to the host pass only."""
    os.makedirs(OBJ, exist_ok=True)
    kernels = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in kernels):
        build()
    obj = os.path.join(OBJ, "abi_hostsan.o")
    host_only = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        host_only += ["-Xarch_host", f]
    cmd = [hipcc()] + _flags() + ["-O1", "-g"] + host_only + ["-c", os.path.join(CSRC, "abi.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on abi.cpp (host sanitizers):\n{r.stdout}\n{r.stderr}")
    _link([obj] + kernels, HOSTSAN_LIB)
    return HOSTSAN_LIB


def build(verbose: bool = False) -> str:
    """Compile every source, link libspin.so and libspin_probe.so; returns the
    path of libspin.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(LIB)
        print(PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
