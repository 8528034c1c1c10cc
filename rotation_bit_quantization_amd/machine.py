"""Machine probes through libspin_probe (include/spin_probe.h): the sustained
dense MFMA rate of the hot path's two matrix instructions with the shader
clock meanwhile, and the streaming read bandwidth of HBM.  bench.py reports
them beside the published peaks; nothing in the hot path uses them.

Torch only provides device memory and the stream.
"""

import ctypes
import os

import numpy as np

from .timing import hip_events

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

EXPORTED_SYMBOLS = ("spin_probe_mfma", "spin_probe_read")
OPS_PER_MFMA = {0: 2 * 32 * 32 * 32, 1: 2 * 32 * 32 * 16}     # v_mfma_i32_32x32x32_i8, v_mfma_f32_32x32x16_f16


def library_path() -> str:
    return os.path.join(_HERE, "libspin_probe.so")


def load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with `python -m rotation_bit_quantization_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.spin_probe_mfma.argtypes = [i, i, i, vp, vp, vp]
    lib.spin_probe_read.argtypes = [vp, ctypes.c_size_t, i, vp, vp]
    for name in EXPORTED_SYMBOLS:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _operands(kind, seed=5):
    """64 lanes x 8 dwords of the hot path's kind of data: INT4 codes widened
    x16 into int8 (kind 0), N(0,1) fp16 (kind 1)."""
    rng = np.random.default_rng(seed)
    if kind == 0:
        return (rng.integers(-7, 8, size=64 * 32) * 16).astype(np.int8).view(np.uint32)
    return rng.standard_normal(64 * 16).astype(np.float16).view(np.uint32)


def mfma_rate(kind: int, waves_per_cu: int = 8, iters: int = 20000) -> dict:
    """Sustained rate of one MFMA instruction over the whole chip, in T ops/s,
    with the shader clock (median over waves) while it ran."""
    import torch
    lib = load()
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * waves_per_cu // 4
    ops = torch.from_numpy(_operands(kind)).to(dev)
    timing = torch.zeros(blocks * 4 * 4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    he = hip_events()
    a, b = he.new(), he.new()
    for timed in (False, True):
        if timed:
            he.record(a, stream)
        rc = lib.spin_probe_mfma(kind, blocks, iters, ops.data_ptr(), timing.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"spin_probe_mfma failed ({rc})")
        if timed:
            he.record(b, stream)
    torch.cuda.synchronize()
    ms = he.ms(a, b)
    he.release()
    t = timing.cpu().numpy().reshape(-1, 4).astype(np.float64)
    ghz = np.median((t[:, 1] - t[:, 0]) / ((t[:, 3] - t[:, 2]) / 1e8)) / 1e9
    total = blocks * 4 * 4 * iters * OPS_PER_MFMA[kind]
    return {"tops": total / (ms * 1e-3) / 1e12, "clock_ghz": float(ghz), "ms": ms, "waves": blocks * 4}


def read_bandwidth(nbytes: int = 2 << 30, blocks_per_cu: int = 8) -> dict:
    """Streaming read bandwidth (non-temporal 16-byte loads) over `nbytes`."""
    import torch
    lib = load()
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    buf = torch.full((nbytes // 4,), 0x3C003C00, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    he = hip_events()
    times = []
    for rep in range(4):
        a, b = he.new(), he.new()
        he.record(a, stream)
        rc = lib.spin_probe_read(buf.data_ptr(), nbytes, cus * blocks_per_cu, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"spin_probe_read failed ({rc})")
        he.record(b, stream)
        torch.cuda.synchronize()
        if rep:
            times.append(he.ms(a, b))
    he.release()
    del buf
    ms = float(np.median(times))
    return {"tbps": nbytes / (ms * 1e-3) / 1e12, "ms": ms, "bytes": nbytes}
