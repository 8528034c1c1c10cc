"""Thin Python binding of the libspin C ABI (ctypes; argument marshalling only).

Every function here checks tensor dtype / device / contiguity, allocates the
outputs it was not given (torch device memory), and calls the C entry point
of the same name on torch's current HIP stream.  All arithmetic happens in the
HIP kernels of libspin.so; if the library is missing this module raises
instead of computing anything itself.

Declarations and contracts: include/libspin.h.
"""

import ctypes
import os

import torch

__all__ = ["SpinError", "load", "library_path", "SPIN_OK", "SPIN_ERR_NULL",
           "SPIN_ERR_BAD_SHAPE", "SPIN_ERR_MISALIGNED", "SPIN_ERR_UNSUPPORTED", "SPIN_ERR_HIP",
           "SPIN_F32", "SPIN_F16", "spin_status_string", "spin_fold_rotation", "spin_fwht_quant",
           "spin_w4a4_gemm", "spin_kv_quant", "spin_fwht_quant8", "spin_w4a8_gemm", "spin_kv_quant8",
           "spin_kv_qkv", "spin_w4a4_gemm_ex", "spin_fwht_quant_gemm", "spin_fwht_quant_gemm_noalloc", "spin_fwht_quant_f6", "spin_w4a4_gemm_f6",
           "spin_codes_f6", "spin_w4a4_gemm_f6f6", "f6_bytes", "SPIN_GEMM_AUTO", "SPIN_GEMM_INT8", "SPIN_GEMM_FP6", "SPIN_GEMM_FP6_SPLITK",
           "EXPORTED_SYMBOLS"]

SPIN_OK, SPIN_ERR_NULL, SPIN_ERR_BAD_SHAPE, SPIN_ERR_MISALIGNED, SPIN_ERR_UNSUPPORTED, \
    SPIN_ERR_HIP = range(6)
SPIN_F32, SPIN_F16 = 0, 1
SPIN_GEMM_AUTO, SPIN_GEMM_INT8, SPIN_GEMM_FP6, SPIN_GEMM_FP6_SPLITK = 0, 1, 2, 3
SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS = 1025

EXPORTED_SYMBOLS = ("spin_fold_rotation", "spin_fwht_quant", "spin_w4a4_gemm", "spin_kv_quant",
                    "spin_fwht_quant8", "spin_w4a8_gemm", "spin_kv_quant8", "spin_kv_qkv", "spin_w4a4_gemm_ex",
                    "spin_fwht_quant_gemm", "spin_fwht_quant_gemm_noalloc", "spin_fwht_quant_f6",
                    "spin_w4a4_gemm_f6", "spin_codes_f6", "spin_w4a4_gemm_f6f6",
                    "spin_status_string", "spin_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path() -> str:
    """The in-tree libspin.so, or the build SPIN_LIBRARY names (the
    host-sanitized one of the sanitizer tests); there is no other fallback."""
    return os.environ.get("SPIN_LIBRARY") or os.path.join(_HERE, "libspin.so")


class SpinError(RuntimeError):
    """A libspin call returned a non-zero spin_status."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {spin_status_string(status)}")


def load():
    """Load libspin.so (raises OSError with a build hint if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with `python -m rotation_bit_quantization_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.spin_fold_rotation.argtypes = [vp, i, i, vp, i, vp, vp, vp, vp]
    lib.spin_fwht_quant.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
    lib.spin_w4a4_gemm.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp, vp]
    lib.spin_w4a4_gemm_ex.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp, i, vp]
    lib.spin_fwht_quant_gemm.argtypes = [vp, i, i, i, i, vp, vp, i, vp, vp, vp, vp, vp, vp]
    lib.spin_fwht_quant_gemm_noalloc.argtypes = [vp, i, i, i, i, vp, vp, i, vp, vp, vp, vp, vp]
    lib.spin_fwht_quant_f6.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
    lib.spin_w4a4_gemm_f6.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, vp, vp]
    lib.spin_codes_f6.argtypes = [vp, i, i, vp, vp, vp]
    lib.spin_w4a4_gemm_f6f6.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, vp, vp, vp]
    lib.spin_kv_quant.argtypes = [vp, i, i, i, i, i, vp, vp, vp, vp]
    lib.spin_fwht_quant8.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
    lib.spin_w4a8_gemm.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp, vp]
    lib.spin_kv_quant8.argtypes = [vp, i, i, i, i, i, vp, vp, vp, vp]
    lib.spin_kv_qkv.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp]
    for name in ("spin_fold_rotation", "spin_fwht_quant", "spin_w4a4_gemm", "spin_kv_quant",
                 "spin_fwht_quant8", "spin_w4a8_gemm", "spin_kv_quant8", "spin_kv_qkv", "spin_w4a4_gemm_ex", "spin_fwht_quant_gemm",
                 "spin_fwht_quant_gemm_noalloc", "spin_fwht_quant_f6", "spin_w4a4_gemm_f6"):
        getattr(lib, name).restype = ctypes.c_int
    lib.spin_status_string.argtypes = [ctypes.c_int]
    lib.spin_status_string.restype = ctypes.c_char_p
    lib.spin_version.argtypes = []
    lib.spin_version.restype = ctypes.c_int
    _lib = lib
    return lib


def spin_status_string(status: int) -> str:
    return load().spin_status_string(int(status)).decode()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    """The hipStream_t to launch on, as an integer: torch's current stream on the
    current device unless one is given."""
    if stream is None:
        if _raw_stream is not None and _cur_device is not None:
            return _raw_stream(_cur_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtypes, shape=None):
    """Raise unless t is a contiguous GPU tensor of one of `dtypes` (and `shape`)."""
    try:
        if t.is_cuda and t.dtype in dtypes and (shape is None or t.shape == shape) and t.is_contiguous():
            return
    except AttributeError:
        pass
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(fn, status):
    if status != SPIN_OK:
        raise SpinError(fn, status)


def _dtype_code(t):
    return SPIN_F16 if t.dtype == torch.float16 else SPIN_F32


def spin_fold_rotation(W, R, r_block, W_rot=None, Wq=None, w_scale=None, stream=None):
    """W [K, N] fp32, R [r, r] fp32 or None -> (W_rot [K, N] fp32, Wq [N, K/2] u8, w_scale [N] fp32)."""
    _check(W, "W", (torch.float32,))
    K, N = W.shape
    if R is not None:
        _check(R, "R", (torch.float32,), (r_block, r_block))
    dev = W.device
    W_rot = torch.empty((K, N), dtype=torch.float32, device=dev) if W_rot is None else W_rot
    Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev) if Wq is None else Wq
    w_scale = torch.empty((N,), dtype=torch.float32, device=dev) if w_scale is None else w_scale
    _check(W_rot, "W_rot", (torch.float32,), (K, N))
    _check(Wq, "Wq", (torch.uint8,), (N, K // 2))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    st = load().spin_fold_rotation(_ptr(W), K, N, _ptr(R), int(r_block), _ptr(W_rot), _ptr(Wq),
                                   _ptr(w_scale), _stream(stream))
    _raise("spin_fold_rotation", st)
    return W_rot, Wq, w_scale


def spin_fwht_quant(X, had_n, Xq=None, x_scale=None, X_rot=None, want_rot=False, stream=None):
    """X [M, K] fp16/fp32 -> (Xq [M, K/2] u8, x_scale [M] fp32, X_rot [M, K] fp32 or None)."""
    _check(X, "X", (torch.float16, torch.float32))
    M, K = X.shape
    dev = X.device
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if Xq is None else Xq
    x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
    if X_rot is None and want_rot:
        X_rot = torch.empty((M, K), dtype=torch.float32, device=dev)
    _check(Xq, "Xq", (torch.uint8,), (M, K // 2))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    if X_rot is not None:
        _check(X_rot, "X_rot", (torch.float32,), (M, K))
    st = load().spin_fwht_quant(_ptr(X), _dtype_code(X), M, K, int(had_n), _ptr(Xq), _ptr(x_scale),
                                _ptr(X_rot), _stream(stream))
    _raise("spin_fwht_quant", st)
    return Xq, x_scale, X_rot


def spin_w4a4_gemm(Xq, x_scale, Wq, w_scale, Y=None, acc_out=None, want_acc=False, kernel=None,
                   stream=None):
    """Packed Xq [M, K/2], Wq [N, K/2] + scales -> (Y [M, N] fp32, acc [M, N] int32 or None).

    ``kernel`` (SPIN_GEMM_INT8 / SPIN_GEMM_FP6 / SPIN_GEMM_FP6_SPLITK) names the kernel family through
    spin_w4a4_gemm_ex; None leaves the choice to the library."""
    _check(Xq, "Xq", (torch.uint8,))
    _check(Wq, "Wq", (torch.uint8,))
    M, Kh = Xq.shape
    N, Kh2 = Wq.shape
    if Kh != Kh2:
        raise ValueError("Xq and Wq disagree on K")
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    dev = Xq.device
    Y = torch.empty((M, N), dtype=torch.float32, device=dev) if Y is None else Y
    if acc_out is None and want_acc:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check(Y, "Y", (torch.float32,), (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", (torch.int32,), (M, N))
    if kernel is None:
        st = load().spin_w4a4_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, 2 * Kh,
                                   _ptr(Y), _ptr(acc_out), _stream(stream))
        _raise("spin_w4a4_gemm", st)
    else:
        st = load().spin_w4a4_gemm_ex(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, 2 * Kh,
                                      _ptr(Y), _ptr(acc_out), int(kernel), _stream(stream))
        _raise("spin_w4a4_gemm_ex", st)
    return Y, acc_out


def f6_bytes(M, K):
    """Bytes of an [M][K] activation code matrix in the FP6 operand layout."""
    return ((M + 31) // 32) * (K // 64) * 1536


def spin_fwht_quant_f6(X, Xf6=None, x_sum=None, x_scale=None, stream=None, had_n=12288):
    """X [M, K] -> (Xf6 uint8 [f6_bytes(M, K)], x_sum [M] int32, x_scale [M] fp32).

    had_n = 12288: X fp16 [M, 12288], the R4 Hadamard first; had_n = 1: X fp16 / fp32, quantized as given."""
    _check(X, "X", (torch.float16,) if had_n == 12288 else (torch.float16, torch.float32))
    M, K = X.shape
    dev = X.device
    Xf6 = torch.empty((f6_bytes(M, K),), dtype=torch.uint8, device=dev) if Xf6 is None else Xf6
    x_sum = torch.empty((M,), dtype=torch.int32, device=dev) if x_sum is None else x_sum
    x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
    _check(Xf6, "Xf6", (torch.uint8,), (f6_bytes(M, K),))
    _check(x_sum, "x_sum", (torch.int32,), (M,))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    st = load().spin_fwht_quant_f6(_ptr(X), _dtype_code(X), M, K, int(had_n), _ptr(Xf6), _ptr(x_sum),
                                   _ptr(x_scale), _stream(stream))
    _raise("spin_fwht_quant_f6", st)
    return Xf6, x_sum, x_scale


def spin_w4a4_gemm_f6(Xf6, x_sum, x_scale, Wq, w_scale, Y=None, acc_out=None, want_acc=False, stream=None):
    """Activation codes in the FP6 operand layout (+ row sums, scales) x packed Wq [N, K/2]
    -> (Y [M, N] fp32, acc [M, N] int32 or None)."""
    _check(x_sum, "x_sum", (torch.int32,))
    M = x_sum.shape[0]
    _check(Wq, "Wq", (torch.uint8,))
    N, Kh = Wq.shape
    K = 2 * Kh
    _check(Xf6, "Xf6", (torch.uint8,), (f6_bytes(M, K),))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    dev = Wq.device
    Y = torch.empty((M, N), dtype=torch.float32, device=dev) if Y is None else Y
    if acc_out is None and want_acc:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check(Y, "Y", (torch.float32,), (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", (torch.int32,), (M, N))
    st = load().spin_w4a4_gemm_f6(_ptr(Xf6), _ptr(x_sum), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, K,
                                  _ptr(Y), _ptr(acc_out), _stream(stream))
    _raise("spin_w4a4_gemm_f6", st)
    return Y, acc_out


def spin_codes_f6(Wq, Wf6=None, w_sum=None, stream=None):
    """Packed codes [N, K/2] (weights, or activations) -> (uint8 [f6_bytes(N, K)], row sums [N] int32):
    the codes in the FP6 operand layout, for spin_w4a4_gemm_f6f6."""
    _check(Wq, "Wq", (torch.uint8,))
    N, Kh = Wq.shape
    K = 2 * Kh
    dev = Wq.device
    Wf6 = torch.empty((f6_bytes(N, K),), dtype=torch.uint8, device=dev) if Wf6 is None else Wf6
    w_sum = torch.empty((N,), dtype=torch.int32, device=dev) if w_sum is None else w_sum
    _check(Wf6, "Wf6", (torch.uint8,), (f6_bytes(N, K),))
    _check(w_sum, "w_sum", (torch.int32,), (N,))
    st = load().spin_codes_f6(_ptr(Wq), N, K, _ptr(Wf6), _ptr(w_sum), _stream(stream))
    _raise("spin_codes_f6", st)
    return Wf6, w_sum


def spin_w4a4_gemm_f6f6(Xf6, x_sum, x_scale, Wf6, w_sum, w_scale, K, Y=None, acc_out=None, want_acc=False,
                        stream=None):
    """Both operands in the FP6 operand layout (+ code sums, scales) -> (Y [M, N] fp32, acc [M, N] int32
    or None).  K is the reduction length (the layouts do not carry it)."""
    _check(x_sum, "x_sum", (torch.int32,))
    _check(w_sum, "w_sum", (torch.int32,))
    M, N = x_sum.shape[0], w_sum.shape[0]
    _check(Xf6, "Xf6", (torch.uint8,), (f6_bytes(M, K),))
    _check(Wf6, "Wf6", (torch.uint8,), (f6_bytes(N, K),))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    dev = Wf6.device
    Y = torch.empty((M, N), dtype=torch.float32, device=dev) if Y is None else Y
    if acc_out is None and want_acc:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check(Y, "Y", (torch.float32,), (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", (torch.int32,), (M, N))
    st = load().spin_w4a4_gemm_f6f6(_ptr(Xf6), _ptr(x_sum), _ptr(x_scale), _ptr(Wf6), _ptr(w_sum), _ptr(w_scale),
                                    M, N, K, _ptr(Y), _ptr(acc_out), _stream(stream))
    _raise("spin_w4a4_gemm_f6f6", st)
    return Y, acc_out


_workspaces = {}


def fused_workspace(device):
    """The zero-initialised workspace spin_fwht_quant_gemm needs, one per device
    (each call leaves it zero; calls sharing it must not overlap)."""
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS, dtype=torch.int32, device=dev)
        _workspaces[key] = ws
    return ws


def spin_fwht_quant_gemm(X, Wq, w_scale, Xq=None, x_scale=None, Y=None, acc_out=None, want_acc=False,
                         workspace=None, stream=None):
    """X [M, 12288] fp16 (R4 = H_12288 applied online) and the folded Wq [N, 6144], w_scale [N]
    -> (Y [M, N] fp32, Xq [M, 6144] u8, x_scale [M] fp32, acc [M, N] int32 or None), one launch."""
    _check(X, "X", (torch.float16,))
    _check(Wq, "Wq", (torch.uint8,))
    M, K = X.shape
    N = Wq.shape[0]
    _check(Wq, "Wq", (torch.uint8,), (N, K // 2))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    dev = X.device
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if Xq is None else Xq
    x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
    Y = torch.empty((M, N), dtype=torch.float32, device=dev) if Y is None else Y
    if acc_out is None and want_acc:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check(Xq, "Xq", (torch.uint8,), (M, K // 2))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    _check(Y, "Y", (torch.float32,), (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", (torch.int32,), (M, N))
    ws = fused_workspace(dev) if workspace is None else workspace
    _check(ws, "workspace", (torch.int32,), (SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS,))
    st = load().spin_fwht_quant_gemm(_ptr(X), SPIN_F16, M, K, K, _ptr(Wq), _ptr(w_scale), N, _ptr(Xq),
                                     _ptr(x_scale), _ptr(Y), _ptr(acc_out), _ptr(ws), _stream(stream))
    _raise("spin_fwht_quant_gemm", st)
    return Y, Xq, x_scale, acc_out


def spin_fwht_quant_gemm_noalloc(X, Wq, w_scale, Xq, x_scale, Y, acc_out=None, stream=None):
    """spin_fwht_quant_gemm into caller-given outputs, with the library's own flags:
    the call allocates nothing (every tensor is passed in)."""
    _check(X, "X", (torch.float16,))
    M, K = X.shape
    N = Wq.shape[0]
    _check(Wq, "Wq", (torch.uint8,), (N, K // 2))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    _check(Xq, "Xq", (torch.uint8,), (M, K // 2))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    _check(Y, "Y", (torch.float32,), (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", (torch.int32,), (M, N))
    st = load().spin_fwht_quant_gemm_noalloc(_ptr(X), SPIN_F16, M, K, K, _ptr(Wq), _ptr(w_scale), N, _ptr(Xq),
                                             _ptr(x_scale), _ptr(Y), _ptr(acc_out), _stream(stream))
    _raise("spin_fwht_quant_gemm_noalloc", st)
    return Y, Xq, x_scale, acc_out


def spin_kv_quant(X, rotate, quantize=True, codes=None, scale=None, X_rot=None, want_rot=False,
                  stream=None):
    """X [T, H, 128] fp16/fp32 -> (codes [T, H, 64] u8 | None, scale [T, H] fp16 | None, X_rot | None).

    ``scale`` is returned as a float16 tensor holding the fp16 bit patterns the
    library writes.
    """
    _check(X, "X", (torch.float16, torch.float32))
    T, H, D = X.shape
    dev = X.device
    if quantize:
        codes = torch.empty((T, H, D // 2), dtype=torch.uint8, device=dev) if codes is None else codes
        scale = torch.empty((T, H), dtype=torch.float16, device=dev) if scale is None else scale
        _check(codes, "codes", (torch.uint8,), (T, H, D // 2))
        _check(scale, "scale", (torch.float16,), (T, H))
    if X_rot is None and (want_rot or not quantize):
        X_rot = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    if X_rot is not None:
        _check(X_rot, "X_rot", (torch.float32,), (T, H, D))
    st = load().spin_kv_quant(_ptr(X), _dtype_code(X), T, H, D, int(rotate), _ptr(codes),
                              _ptr(scale), _ptr(X_rot), _stream(stream))
    _raise("spin_kv_quant", st)
    return codes, scale, X_rot


# ---------------------------------------------------------------- W4A8KV8 variant

def spin_fwht_quant8(X, had_n, Xq8=None, x_scale=None, X_rot=None, want_rot=False, stream=None):
    """X [M, K] fp16/fp32 -> (Xq8 [M, K] int8, x_scale [M] fp32, X_rot [M, K] fp32 or None)."""
    _check(X, "X", (torch.float16, torch.float32))
    M, K = X.shape
    dev = X.device
    Xq8 = torch.empty((M, K), dtype=torch.int8, device=dev) if Xq8 is None else Xq8
    x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
    if X_rot is None and want_rot:
        X_rot = torch.empty((M, K), dtype=torch.float32, device=dev)
    _check(Xq8, "Xq8", (torch.int8,), (M, K))
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    if X_rot is not None:
        _check(X_rot, "X_rot", (torch.float32,), (M, K))
    st = load().spin_fwht_quant8(_ptr(X), _dtype_code(X), M, K, int(had_n), _ptr(Xq8), _ptr(x_scale),
                                 _ptr(X_rot), _stream(stream))
    _raise("spin_fwht_quant8", st)
    return Xq8, x_scale, X_rot


def spin_w4a8_gemm(Xq8, x_scale, Wq, w_scale, Y=None, acc_out=None, want_acc=False, stream=None):
    """Int8 Xq8 [M, K], packed Wq [N, K/2] + scales -> (Y [M, N] fp32, acc [M, N] int32 or None)."""
    _check(Xq8, "Xq8", (torch.int8,))
    _check(Wq, "Wq", (torch.uint8,))
    M, K = Xq8.shape
    N, Kh = Wq.shape
    if K != 2 * Kh:
        raise ValueError("Xq8 and Wq disagree on K")
    _check(x_scale, "x_scale", (torch.float32,), (M,))
    _check(w_scale, "w_scale", (torch.float32,), (N,))
    dev = Xq8.device
    Y = torch.empty((M, N), dtype=torch.float32, device=dev) if Y is None else Y
    if acc_out is None and want_acc:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=dev)
    _check(Y, "Y", (torch.float32,), (M, N))
    if acc_out is not None:
        _check(acc_out, "acc_out", (torch.int32,), (M, N))
    st = load().spin_w4a8_gemm(_ptr(Xq8), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, K,
                               _ptr(Y), _ptr(acc_out), _stream(stream))
    _raise("spin_w4a8_gemm", st)
    return Y, acc_out


def spin_kv_quant8(X, rotate, quantize=True, codes=None, scale=None, X_rot=None, want_rot=False,
                   stream=None):
    """X [T, H, 128] fp16/fp32 -> (codes [T, H, 128] int8 | None, scale [T, H] fp16 | None, X_rot | None)."""
    _check(X, "X", (torch.float16, torch.float32))
    T, H, D = X.shape
    dev = X.device
    if quantize:
        codes = torch.empty((T, H, D), dtype=torch.int8, device=dev) if codes is None else codes
        scale = torch.empty((T, H), dtype=torch.float16, device=dev) if scale is None else scale
        _check(codes, "codes", (torch.int8,), (T, H, D))
        _check(scale, "scale", (torch.float16,), (T, H))
    if X_rot is None and (want_rot or not quantize):
        X_rot = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    if X_rot is not None:
        _check(X_rot, "X_rot", (torch.float32,), (T, H, D))
    st = load().spin_kv_quant8(_ptr(X), _dtype_code(X), T, H, D, int(rotate), _ptr(codes),
                               _ptr(scale), _ptr(X_rot), _stream(stream))
    _raise("spin_kv_quant8", st)
    return codes, scale, X_rot


def spin_kv_qkv(K, V, Q=None, bits=4, want_k_rot=False, out=None, stream=None):
    """One launch for a layer's KV step: K [T, Hkv, 128] rotated + quantized, V [T, Hkv, 128]
    quantized, Q [T, Hq, 128] (optional) rotated.

    Returns a dict with ``K_codes``, ``K_scale``, ``V_codes``, ``V_scale`` (scales as float16
    tensors holding the fp16 bit patterns), ``Q_rot`` (or None) and ``K_rot`` (or None).
    Codes are [T, Hkv, 64] uint8 at bits=4 and [T, Hkv, 128] int8 at bits=8.  ``out`` may
    hold preallocated tensors under the same names; missing ones are allocated.
    """
    _check(K, "K", (torch.float16, torch.float32))
    T, Hkv, D = K.shape
    _check(V, "V", (K.dtype,), (T, Hkv, D))
    Hq = 0
    if Q is not None:
        _check(Q, "Q", (K.dtype,))
        if Q.dim() != 3 or Q.shape[0] != T or Q.shape[2] != D:
            raise ValueError(f"Q has shape {tuple(Q.shape)}, expected ({T}, Hq, {D})")
        Hq = Q.shape[1]
    dev = K.device
    if bits == 4:
        cshape, cdtype = (T, Hkv, D // 2), torch.uint8
    elif bits == 8:
        cshape, cdtype = (T, Hkv, D), torch.int8
    else:
        raise ValueError("bits must be 4 or 8")
    want = {
        "K_codes": (cshape, cdtype),
        "K_scale": ((T, Hkv), torch.float16),
        "V_codes": (cshape, cdtype),
        "V_scale": ((T, Hkv), torch.float16),
    }
    if Q is not None:
        want["Q_rot"] = ((T, Hq, D), torch.float32)
    if want_k_rot:
        want["K_rot"] = ((T, Hkv, D), torch.float32)
    given = dict(out or {})
    res = {"Q_rot": None, "K_rot": None}
    for name, (shape, dtype) in want.items():
        t = given.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
        _check(t, name, (dtype,), shape)
        res[name] = t
    st = load().spin_kv_qkv(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(K), T, Hq, Hkv, D, int(bits),
                            _ptr(res["Q_rot"]), _ptr(res["K_codes"]), _ptr(res["K_scale"]),
                            _ptr(res["K_rot"]), _ptr(res["V_codes"]), _ptr(res["V_scale"]), _stream(stream))
    _raise("spin_kv_qkv", st)
    return res
