"""Thin ctypes binding of the test-support library ``libmoe_harness.so`` (C
ABI in ``include/moe_harness.h``): the expert stand-in, the exchange
stand-in and the bandwidth probes.  None of them is on the data path.  Same
names as the C entry points; arguments are checked and marshalled as in
``binding.py``, and a missing library is an error."""
from __future__ import annotations

import ctypes
import os

import torch

from .binding import (RecvLayout, _check, _ptr, _stream, _want, _want_offsets, _want_rows,
                      _want_scales)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_harness.so")

EXPORTS = ("moe_expert_standin", "moe_exchange_blocks", "moe_stream_probe")

MOE_PROBE_COPY = 0
MOE_PROBE_READ_CACHED = 1
MOE_PROBE_READ_STREAM = 2

_lib = None


def load() -> ctypes.CDLL:
    """Load the built test-support library (never builds)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.moe_expert_standin.argtypes = [P, P, i32, P, i32, i64, i32, i32, P, P, P]
    lib.moe_exchange_blocks.argtypes = [P, P, i64, P, P, i64, i32, i32, P, i32, i32, P, i32, P]
    lib.moe_stream_probe.argtypes = [P, P, sz, i32, P]
    for n in EXPORTS:
        getattr(lib, n).restype = i32
    _lib = lib
    return lib


def moe_expert_standin(recv: torch.Tensor, recv_scales: torch.Tensor | None, quant_in: int,
                       expert_offsets: torch.Tensor, E: int, max_rows: int, H: int,
                       quant_out: int, ret: torch.Tensor, ret_scales: torch.Tensor | None,
                       stream=None) -> None:
    _want(expert_offsets, torch.int32, "expert_offsets")
    _want_scales(recv_scales, max_rows, quant_in, "recv_scales")
    _want_scales(ret_scales, max_rows, quant_out, "ret_scales")
    _check("moe_expert_standin",
           load().moe_expert_standin(_ptr(recv), _ptr(recv_scales), quant_in,
                                     _ptr(expert_offsets), E, max_rows, H, quant_out, _ptr(ret),
                                     _ptr(ret_scales), _stream(stream)))


def moe_exchange_blocks(send: torch.Tensor, send_scales: torch.Tensor | None, source_rows: int,
                        recv: torch.Tensor, recv_scales: torch.Tensor | None, max_rows: int,
                        H: int, quant: int, src_offsets: torch.Tensor, E: int, R: int,
                        rl: RecvLayout, reverse: bool = False, stream=None) -> None:
    _want_offsets(src_offsets, E, R)
    _want_rows(send, send_scales, R * source_rows, H, quant, "send")
    _want_rows(recv, recv_scales, max_rows, H, quant, "recv")
    _check("moe_exchange_blocks",
           load().moe_exchange_blocks(_ptr(send), _ptr(send_scales), source_rows, _ptr(recv),
                                      _ptr(recv_scales), max_rows, H, quant, _ptr(src_offsets),
                                      E, R, _ptr(rl.recv_offsets), 1 if reverse else 0,
                                      _stream(stream)))


def moe_stream_probe(src: torch.Tensor, dst: torch.Tensor, nbytes: int, mode: int,
                     stream=None) -> None:
    """Copy (dst = src over nbytes) or read sweep of src (dst: a uint32 that
    receives the count of all-ones 16-byte vectors)."""
    need = nbytes if mode == MOE_PROBE_COPY else 4
    if src.numel() * src.element_size() < nbytes or dst.numel() * dst.element_size() < need:
        raise ValueError("probe buffers smaller than the sweep")
    _check("moe_stream_probe",
           load().moe_stream_probe(_ptr(src), _ptr(dst), nbytes, mode, _stream(stream)))
