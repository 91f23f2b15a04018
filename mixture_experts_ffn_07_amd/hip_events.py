"""HIP events through the HIP runtime already loaded in the process (ctypes).

Used by the benchmark to bracket single kernel launches inside the library
(see moe_profile_kernel) and read their durations."""
from __future__ import annotations

import ctypes
import re

_hip = None


def _runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (the runtime torch loaded is the one the library uses)
        path = None
        for line in open("/proc/self/maps"):
            m = re.search(r"(\S*libamdhip64\.so\S*)", line)
            if m:
                path = m.group(1)
                break
        _hip = ctypes.CDLL(path or "libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


class HipEvent:
    def __init__(self):
        h = ctypes.c_void_p()
        rc = _runtime().hipEventCreate(ctypes.byref(h))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.handle = h.value

    def synchronize(self) -> None:
        _runtime().hipEventSynchronize(self.handle)

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _runtime().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle and _hip is not None:
                _hip.hipEventDestroy(self.handle)
        except Exception:
            pass
