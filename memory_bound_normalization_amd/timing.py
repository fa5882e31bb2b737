"""Timing events for GPU measurements (bench.py and the probe tools)."""

from __future__ import annotations

import ctypes


class HipTimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    A default event record performs a system-scope release (an L2 writeback and
    invalidate) when it completes; the HIP header documents this flag for
    events used only to measure time, to avoid that cost and its effect on
    the following work. Measured on MI355X around each 170 us RMSNorm launch:
    default events (torch's) read 170.8 us, these 169.1 us, the rocprofv3
    kernel trace 166.4 us. Recorded on the stream the kernels run on.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream):
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")  # already loaded by torch
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        self.events = []

    def new(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.events.append(e)
        return e

    def record(self, e):
        rc = self.hip.hipEventRecord(e, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []
