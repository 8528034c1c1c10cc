"""Kernel timing with HIP events of the runtime the process already uses
(PyTorch's), created with hipEventDisableSystemFence.

Default HIP events (what torch.cuda.Event records) release to system scope at
every record, which writes the cache back and slows the kernels between the
events; these do not.  They are recorded on the stream the kernels are
launched on.
"""

import ctypes

DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self._hip = ctypes.CDLL(path or "libamdhip64.so.7")
        self._made = []

    def new(self):
        ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self._made.append(ev)
        return ev

    def record(self, ev, stream):
        rc = self._hip.hipEventRecord(ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value

    def release(self):
        for ev in self._made:
            self._hip.hipEventDestroy(ev)
        self._made = []


_EVENTS = None


def hip_events() -> HipEvents:
    """The process-wide event helper (created on first use, after torch has
    loaded the HIP runtime)."""
    global _EVENTS
    if _EVENTS is None:
        _EVENTS = HipEvents()
    return _EVENTS
