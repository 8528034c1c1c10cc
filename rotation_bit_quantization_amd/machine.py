"""Machine probes through libspin_probe (include/spin_probe.h): the sustained
dense MFMA rate of the hot path's three matrix instructions with the shader
clock meanwhile, the streaming read bandwidth of HBM, and the LDS throughput
of one compute unit in the FP6 GEMM's access patterns.  bench.py reports
them beside the published peaks; nothing in the hot path uses them.

Torch only provides device memory and the stream.
"""

import ctypes
import os

import numpy as np

from .timing import hip_events

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

EXPORTED_SYMBOLS = ("spin_probe_mfma", "spin_probe_read", "spin_probe_lds")
# v_mfma_i32_32x32x32_i8, v_mfma_f32_32x32x16_f16, v_mfma_scale_f32_32x32x64_f8f6f4 (FP6)
OPS_PER_MFMA = {0: 2 * 32 * 32 * 32, 1: 2 * 32 * 32 * 16, 2: 2 * 32 * 32 * 64}


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
    lib.spin_probe_lds.argtypes = [i, i, i, vp, vp, vp]
    for name in EXPORTED_SYMBOLS:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _fp6_fields(u):
    """32 unsigned 6-bit fields -> six little-endian dwords (field f at bits
    6f .. 6f + 5 of the 192-bit operand)."""
    v = 0
    for f, x in enumerate(u):
        v |= int(x) << (6 * f)
    return [(v >> (32 * i)) & 0xFFFFFFFF for i in range(6)]


def _operands(kind, seed=5):
    """The hot path's kind of data for one wave: INT4 codes widened x16 into
    int8 (kind 0, 64 lanes x 8 dwords), N(0,1) fp16 (kind 1, 64 x 8), INT4
    codes as FP6 E2M3 fields u = q + 8 (kind 2, 64 x 16: A in dwords 0-5, B in
    8-13)."""
    rng = np.random.default_rng(seed)
    if kind == 0:
        return (rng.integers(-7, 8, size=64 * 32) * 16).astype(np.int8).view(np.uint32)
    if kind == 2:
        out = np.zeros((64, 16), np.uint32)
        for lane in range(64):
            out[lane, 0:6] = _fp6_fields(rng.integers(-7, 8, size=32) + 8)
            out[lane, 8:14] = _fp6_fields(rng.integers(-7, 8, size=32) + 8)
        return out.reshape(-1)
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


LDS_BYTES_PER_ROUND = 48          # per thread, every mode


def lds_rate(mode: int, iters: int = 4096) -> dict:
    """LDS bytes per shader cycle of one compute unit (one workgroup of eight
    waves per CU, median over workgroups): mode 0 the FP6 GEMM's operand reads,
    1 its field writes, 2 contiguous 16-byte reads."""
    import torch
    lib = load()
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    timing = torch.zeros(cus * 4, dtype=torch.int64, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        rc = lib.spin_probe_lds(mode, cus, iters, timing.data_ptr(), sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"spin_probe_lds failed ({rc})")
    torch.cuda.synchronize()
    t = timing.cpu().numpy().reshape(-1, 4).astype(np.float64)
    cycles = t[:, 1] - t[:, 0]
    ghz = np.median(cycles / ((t[:, 3] - t[:, 2]) / 1e8)) / 1e9
    per_cu = 512.0 * iters * LDS_BYTES_PER_ROUND / cycles
    return {"bytes_per_clk_per_cu": float(np.median(per_cu)), "clock_ghz": float(ghz)}


def read_floor_us(nbytes: int, sets: int = 4, reps: int = 12, blocks_per_cu: int = 8) -> float:
    """Mean event-timed duration of one streaming read of `nbytes` (rounded
    down to 16) over `sets` buffers used in turn, so that each launch reads
    data that the previous `sets - 1` launches pushed out of the caches: the
    floor a kernel that reads that many bytes from HBM cannot beat when timed
    the same way."""
    import torch
    lib = load()
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes -= nbytes % 16
    bufs = [torch.full((nbytes // 4,), 0x3C003C00, dtype=torch.int32, device=dev) for _ in range(sets)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    he = hip_events()
    ev = [(he.new(), he.new()) for _ in range(reps + sets)]
    for i, (a, b) in enumerate(ev):
        he.record(a, stream)
        rc = lib.spin_probe_read(bufs[i % sets].data_ptr(), nbytes, cus * blocks_per_cu, sink.data_ptr(),
                                 stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"spin_probe_read failed ({rc})")
        he.record(b, stream)
    torch.cuda.synchronize()
    us = float(np.mean([he.ms(a, b) for a, b in ev[sets:]])) * 1e3
    he.release()
    del bufs
    return us


def copy_rate(nbytes: int = 1 << 30) -> dict:
    """Device-to-device copy of `nbytes` (torch's copy kernel): bytes read plus
    bytes written per second, median of four."""
    import torch
    dev = torch.device("cuda")
    src = torch.full((nbytes // 4,), 7, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    he = hip_events()
    times = []
    for rep in range(5):
        a, b = he.new(), he.new()
        he.record(a, stream)
        dst.copy_(src)
        he.record(b, stream)
        torch.cuda.synchronize()
        if rep:
            times.append(he.ms(a, b))
    he.release()
    ms = float(np.median(times))
    return {"tbps": 2 * nbytes / (ms * 1e-3) / 1e12, "ms": ms}
