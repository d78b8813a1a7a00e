"""CU-masked HIP streams: keep the bandwidth-bound dispatch/combine work on a
slice of the compute units so that a concurrent compute kernel (the experts)
keeps the rest.

The ThunderEP write-up (s2.2) rate-limits its communication so that it does
not take all of the memory bandwidth from the concurrent computation.  On one
MI355X the same contention is between kernels of two streams.  Measured with
the dispatch/combine step of the T=16384, H=7168, E=256, k=8 workload (0.62
ms alone) beside a bf16 8192^3 GEMM (0.86-0.88 ms alone): on two ordinary
streams sharing all CUs the pair takes 1.44 ms against 1.48-1.50 ms one after
the other, while confining the data movement to 1/4, 1/2 or 3/4 of the CUs
(the GEMM on the rest) takes 1.69, 1.66-1.67 and 2.84 ms.  The step needs
most CUs to keep enough memory traffic in flight, and the GEMM's matrix work
coexists with it on shared CUs better than on a static partition, so the
masks are an option, not the default.  A plain 1 GiB copy in place of the
step does behave like the write-up's case (slower concurrent than serial on
shared CUs, faster with a quarter/three-quarter split).

Masks: a CU mask is 32-bit words, one bit per CU.  Every word gets a
contiguous run of at least 8 set bits starting at the same bit position, so
every one of the 8 XCDs keeps CUs whether the mask's bits are read as
interleaved across XCDs (bit i -> XCD i mod 8) or as blocks of 32 (bit i ->
XCD i / 32).  Streams are created with the default priority.
"""
from __future__ import annotations

import ctypes
import os

import torch

BITS_PER_WORD = 32
_STEP = 8  # runs are whole multiples of 8 bits: every residue mod 8 is set

_hip = None


def _runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        # the runtime torch loaded; RTLD_NOLOAD refuses to load another copy
        lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        lib.hipExtStreamCreateWithCUMask.argtypes = [
            ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
        lib.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
        lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        lib.hipStreamDestroy.restype = ctypes.c_int
        _hip = lib
    return _hip


def mask_words(num_cus: int, quarters: int, upper: bool = False) -> list[int]:
    """CU mask for `quarters`/4 of the CUs (1, 2 or 3): in every 32-bit word
    the low 8*quarters bits, or with `upper` the other bits of the word (the
    complementary slice)."""
    if quarters not in (1, 2, 3):
        raise ValueError("quarters must be 1, 2 or 3")
    if num_cus <= 0 or num_cus % BITS_PER_WORD:
        raise ValueError("the CU count must be a positive multiple of 32")
    n = quarters * _STEP
    low = (1 << n) - 1
    word = (0xFFFFFFFF & ~low) if upper else low
    return [word] * (num_cus // BITS_PER_WORD)


class CUMaskedStream:
    """A HIP stream restricted to a CU mask, usable as a torch stream
    (``.stream``).  Close it (or use ``with``) once its work is done."""

    def __init__(self, words: list[int], device=None):
        dev = torch.device(device if device is not None else "cuda")
        arr = (ctypes.c_uint32 * len(words))(*words)
        handle = ctypes.c_void_p()
        with torch.cuda.device(dev):
            rc = _runtime().hipExtStreamCreateWithCUMask(ctypes.byref(handle), len(words), arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
        self.words = list(words)
        self._handle = handle
        self.stream = torch.cuda.ExternalStream(handle.value, device=dev)

    def close(self):
        if self._handle is not None:
            self.stream.synchronize()
            _runtime().hipStreamDestroy(self._handle)
            self._handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def split_streams(quarters_for_data: int, device=None):
    """(data stream, compute stream): the data movement on `quarters`/4 of
    the CUs, the compute on the complementary CUs."""
    dev = torch.device(device if device is not None else "cuda")
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    return (CUMaskedStream(mask_words(ncu, quarters_for_data), dev),
            CUMaskedStream(mask_words(ncu, quarters_for_data, upper=True), dev))
