"""Timing events without the system-scope fence.

An event that torch records on a stream also performs a system-scope
release (an L2 writeback and invalidate) before its timestamp is taken;
between two kernels that costs several microseconds of GPU time, and an
event pair around one kernel holds that cost as well as the kernel. HIP's
hipEventDisableSystemFence flag creates events that skip the fence, meant
for events that only measure time. These events come from the HIP runtime
that torch has loaded (the one the library's calls run on), are recorded
on torch streams, and are read only after the caller has synchronised the
device (they do not make the work before them visible to the host).
"""
from __future__ import annotations

import ctypes

import torch

_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip = None


def _runtime():
    """The libamdhip64 this process has loaded (torch's, after CUDA init)."""
    global _hip
    if _hip is None:
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("hip_timing: no HIP runtime is loaded in this process")
        lib = ctypes.CDLL(path)
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for fn in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
            getattr(lib, fn).restype = ctypes.c_int
        _hip = lib
    return _hip


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError("%s failed with HIP error %d" % (what, status))


class FenceFreeEvent:
    """A timing event created with hipEventDisableSystemFence: record() on a
    torch stream, elapsed_time(other) in milliseconds once both have
    completed (after a device synchronisation)."""

    def __init__(self):
        self._lib = _runtime()
        h = ctypes.c_void_p()
        _check(self._lib.hipEventCreateWithFlags(ctypes.byref(h), _HIP_EVENT_DISABLE_SYSTEM_FENCE),
               "hipEventCreateWithFlags")
        self._h = h

    def record(self, stream: torch.cuda.Stream = None):
        st = stream if stream is not None else torch.cuda.current_stream()
        _check(self._lib.hipEventRecord(self._h, ctypes.c_void_p(st.cuda_stream)), "hipEventRecord")

    def elapsed_time(self, end: "FenceFreeEvent") -> float:
        ms = ctypes.c_float()
        _check(self._lib.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h), "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.hipEventDestroy(self._h)
            self._h = None


def record(stream: torch.cuda.Stream = None) -> FenceFreeEvent:
    """A new fence-free event, recorded on `stream` (the current stream)."""
    e = FenceFreeEvent()
    e.record(stream)
    return e
