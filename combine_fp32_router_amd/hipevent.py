"""HIP events without the system-scope fence.

torch.cuda.Event records with a system-scope release: on MI355X that writes
back and invalidates the caches at every record, which shows up as a ~10 us
bubble before the next kernel on the stream.  Timing and same-device
cross-stream ordering need only a device-scope release, so this module
creates events with ``hipEventDisableSystemFence`` through the HIP runtime
that torch has already loaded (same library, looked up by soname, never a
second copy).

Plumbing only: nothing here touches the data path's arithmetic.
"""
from __future__ import annotations

import ctypes
import os

import torch

HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

_hip = None


def _runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        torch.cuda.init()
        # the runtime torch loaded; RTLD_NOLOAD refuses to load another copy
        lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        P = ctypes.c_void_p
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [P, P]
        lib.hipStreamWaitEvent.argtypes = [P, P, ctypes.c_uint]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        lib.hipEventSynchronize.argtypes = [P]
        lib.hipEventDestroy.argtypes = [P]
        for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipStreamWaitEvent",
                  "hipEventElapsedTime", "hipEventSynchronize", "hipEventDestroy"):
            getattr(lib, f).restype = ctypes.c_int
        _hip = lib
    return _hip


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with hipError {rc}")


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


class Event:
    """A HIP event with a device-scope release.  timing=False also disables
    timestamps (pure ordering between streams of one device)."""

    def __init__(self, timing: bool = False):
        lib = _runtime()
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else HIP_EVENT_DISABLE_TIMING)
        self._ev = ctypes.c_void_p()
        _check(lib.hipEventCreateWithFlags(ctypes.byref(self._ev), flags), "hipEventCreateWithFlags")
        self._lib = lib

    def record(self, stream=None):
        _check(self._lib.hipEventRecord(self._ev, _stream_handle(stream)), "hipEventRecord")

    def wait(self, stream=None):
        """Make `stream` wait for this event (no host synchronization)."""
        _check(self._lib.hipStreamWaitEvent(_stream_handle(stream), self._ev, 0), "hipStreamWaitEvent")

    def synchronize(self):
        _check(self._lib.hipEventSynchronize(self._ev), "hipEventSynchronize")

    def elapsed_ms(self, end: "Event") -> float:
        ms = ctypes.c_float(0.0)
        _check(self._lib.hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev), "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        try:
            if self._ev and self._lib is not None:
                self._lib.hipEventDestroy(self._ev)
        except Exception:
            pass
