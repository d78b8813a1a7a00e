"""Thin ctypes binding of ``libmoe_route.so`` (C ABI in ``include/moe_route.h``
and ``include/moe_recv.h``; the test-support library of
``include/moe_harness.h`` has its own binding, ``harness.py``).

Same names as the C entry points; each function only checks that torch
tensors have the dtype, device and contiguity the ABI expects, passes their
device pointers and the stream handle, and raises ``MoeError`` on a non-zero
status.  Every step of the path runs in the HIP kernels; there is no CPU or
PyTorch fallback, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_route.so")

MOE_QUANT_BF16 = 0
MOE_QUANT_INT8 = 1
MOE_QUANT_INT4 = 2
MOE_QUANT_FP8 = 3
MOE_PACK_STREAM = 0x100  # OR into the quant of the pack calls: streaming row stores

EXPORTS = ("moe_route_topk", "moe_dispatch_layout", "moe_dispatch_layout_chunks",
           "moe_route_layout_chunks", "moe_route_layout_chunks_noalloc",
           "moe_dispatch_pack", "moe_combine", "moe_combine_pack", "moe_status_string",
           "moe_row_bytes", "moe_recv_layout", "moe_recv_regroup", "moe_recv_ungroup")

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the built library (never builds, never falls back)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.moe_route_topk.argtypes = [P, i64, i32, i32, P, P, P]
    lib.moe_dispatch_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                        ctypes.POINTER(sz), P]
    lib.moe_dispatch_layout_chunks.argtypes = [P, i64, i64, i32, i32, i32, i32, P, P, P, P, P, P,
                                               P, P, ctypes.POINTER(sz), P]
    lib.moe_route_layout_chunks.argtypes = [P, i64, i64, i32, i32, i32, i32, P, P, P, P, P, P,
                                            P, P, P, P, ctypes.POINTER(sz), P]
    lib.moe_route_layout_chunks_noalloc.argtypes = [P, i64, i64, i32, i32, i32, i32, P, P, P, P,
                                                    P, P, P, P, P, P]
    lib.moe_dispatch_pack.argtypes = [P, i64, i32, i32, P, i32, P, P, P]
    lib.moe_combine.argtypes = [P, P, i32, P, P, i64, i32, i32, P, P]
    lib.moe_combine_pack.argtypes = [P, P, P, P, i64, P, P, P, i64, P, P, i32, i32, i32, P]
    lib.moe_recv_layout.argtypes = [P, i32, i32, i64, P, P, P, P, P, P]
    lib.moe_recv_regroup.argtypes = [P, P, i64, i32, i32, P, P, P, P]
    lib.moe_recv_ungroup.argtypes = [P, P, i64, i32, i32, P, P, P, P]
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_row_bytes.argtypes = [i32, i32]
    lib.moe_row_bytes.restype = i64
    for n in EXPORTS:
        if n not in ("moe_status_string", "moe_row_bytes"):
            getattr(lib, n).restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def moe_row_bytes(H: int, quant: int) -> int:
    """Bytes per row of a row buffer (quantised formats: the codes only; the
    fp32 scale of each row lives in a separate scale array)."""
    return int(load().moe_row_bytes(int(H), int(quant)))


def alloc_rows(rows: int, H: int, quant: int, device) -> tuple[torch.Tensor, torch.Tensor | None]:
    """A row buffer for `rows` rows of format `quant`: (uint8 [rows, row
    bytes], fp32 [rows] scales, or None for bf16)."""
    data = torch.empty((max(rows, 1), moe_row_bytes(H, quant)), dtype=torch.uint8,
                       device=device)[:rows]
    scales = (torch.empty(max(rows, 1), dtype=torch.float32, device=device)[:rows]
              if quant else None)
    return data, scales


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _want(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")


def moe_route_topk(logits: torch.Tensor, k: int, topk_idx: torch.Tensor,
                   topk_w: torch.Tensor, stream=None) -> None:
    """logits fp32 [T, E] -> topk_idx int32 [T, k], topk_w fp32 [T, k]."""
    _want(logits, torch.float32, "logits")
    _want(topk_idx, torch.int32, "topk_idx")
    _want(topk_w, torch.float32, "topk_w")
    T, E = logits.shape
    if topk_idx.numel() != T * k or topk_w.numel() != T * k:
        raise ValueError("topk outputs must hold T*k elements")
    _check("moe_route_topk", load().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx),
                                                   _ptr(topk_w), _stream(stream)))


def layout_workspace_bytes(T: int, E: int, k: int, R: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_dispatch_layout",
           load().moe_dispatch_layout(None, T, E, k, R, 0, None, None, None, None, None, None,
                                      None, ctypes.byref(n), None))
    return int(n.value)


class Layout(NamedTuple):
    expert_counts: torch.Tensor   # [E]
    expert_offsets: torch.Tensor  # [E+1]
    rank_counts: torch.Tensor     # [R]
    rank_offsets: torch.Tensor    # [R+1]
    pos: torch.Tensor             # [T*k]
    row_src: torch.Tensor         # [T*k]
    workspace: torch.Tensor       # uint8 scratch


def alloc_layout(T: int, E: int, k: int, R: int, device) -> Layout:
    i32 = dict(dtype=torch.int32, device=device)
    ws = layout_workspace_bytes(T, E, k, R)
    return Layout(torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(R, **i32),
                  torch.empty(R + 1, **i32), torch.empty(max(T * k, 1), **i32),
                  torch.empty(max(T * k, 1), **i32),
                  torch.empty(ws, dtype=torch.uint8, device=device))


def moe_dispatch_layout(topk_idx: torch.Tensor, T: int, E: int, k: int, R: int, capacity: int,
                        out: Layout, stream=None) -> Layout:
    _want(topk_idx, torch.int32, "topk_idx")
    if topk_idx.numel() < T * k or out.pos.numel() < T * k or out.row_src.numel() < T * k:
        raise ValueError("layout buffers smaller than T*k")
    n = ctypes.c_size_t(out.workspace.numel())
    _check("moe_dispatch_layout",
           load().moe_dispatch_layout(_ptr(topk_idx), T, E, k, R, int(capacity),
                                      _ptr(out.expert_counts), _ptr(out.expert_offsets),
                                      _ptr(out.rank_counts), _ptr(out.rank_offsets),
                                      _ptr(out.pos), _ptr(out.row_src), _ptr(out.workspace),
                                      ctypes.byref(n), _stream(stream)))
    return out


def layout_chunks_workspace_bytes(T: int, chunk_tokens: int, E: int, k: int, R: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_dispatch_layout_chunks",
           load().moe_dispatch_layout_chunks(None, T, chunk_tokens, E, k, R, 0, None, None, None,
                                             None, None, None, None, None, ctypes.byref(n), None))
    return int(n.value)


def route_layout_workspace_bytes(T: int, chunk_tokens: int, E: int, k: int, R: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_route_layout_chunks",
           load().moe_route_layout_chunks(None, T, chunk_tokens, E, k, R, 0, None, None, None,
                                          None, None, None, None, None, None, None,
                                          ctypes.byref(n), None))
    return int(n.value)


class ChunkLayouts(NamedTuple):
    """Outputs of moe_dispatch_layout_chunks for C chunks of chunk_tokens."""
    expert_counts: torch.Tensor   # [C, E]
    expert_offsets: torch.Tensor  # [C, E+1]
    rank_counts: torch.Tensor     # [C, R]
    rank_offsets: torch.Tensor    # [C, R+1]
    pos: torch.Tensor             # [T*k], chunk-relative rows
    row_src: torch.Tensor         # [T*k], chunk-relative slots
    workspace: torch.Tensor
    chunk_tokens: int
    k: int


def alloc_layout_chunks(T: int, chunk_tokens: int, E: int, k: int, R: int, device,
                        chunks: int = 1) -> ChunkLayouts:
    """Room for ceil(T / chunk_tokens) chunks (at least `chunks` rows); the
    workspace serves moe_dispatch_layout_chunks and moe_route_layout_chunks
    over the whole batch, over its first chunk alone and over the remaining
    chunks (the calls a two-stream driver makes; the fused call's workspace
    depends on the number of tokens it is given)."""
    chunk_tokens = max(1, min(chunk_tokens, max(T, 1)))
    C = max(1, chunks, -(-T // chunk_tokens))
    i32 = dict(dtype=torch.int32, device=device)
    spans = {T, min(T, chunk_tokens), max(T - chunk_tokens, 0)}
    ws = max(max(layout_chunks_workspace_bytes(t, chunk_tokens, E, k, R),
                 route_layout_workspace_bytes(t, chunk_tokens, E, k, R)) for t in spans)
    return ChunkLayouts(torch.empty((C, E), **i32), torch.empty((C, E + 1), **i32),
                        torch.empty((C, R), **i32), torch.empty((C, R + 1), **i32),
                        torch.empty(max(T * k, 1), **i32), torch.empty(max(T * k, 1), **i32),
                        torch.empty(ws, dtype=torch.uint8, device=device), chunk_tokens, k)


def layout_view(lay: ChunkLayouts, c: int, T: int) -> Layout:
    """Chunk c of a ChunkLayouts as a one-chunk Layout (views, no copy)."""
    s0 = c * lay.chunk_tokens * lay.k
    s1 = min(T, (c + 1) * lay.chunk_tokens) * lay.k
    return Layout(lay.expert_counts[c], lay.expert_offsets[c], lay.rank_counts[c],
                  lay.rank_offsets[c], lay.pos[s0:max(s1, s0 + 1)],
                  lay.row_src[s0:max(s1, s0 + 1)], lay.workspace)


def layout_chunks_from(lay: ChunkLayouts, c0: int) -> ChunkLayouts:
    """Chunks c0.. of a ChunkLayouts as their own ChunkLayouts (views)."""
    s0 = c0 * lay.chunk_tokens * lay.k
    return ChunkLayouts(lay.expert_counts[c0:], lay.expert_offsets[c0:], lay.rank_counts[c0:],
                        lay.rank_offsets[c0:], lay.pos[s0:], lay.row_src[s0:], lay.workspace,
                        lay.chunk_tokens, lay.k)


def moe_dispatch_layout_chunks(topk_idx: torch.Tensor, T: int, E: int, k: int, R: int,
                               capacity: int, chunk_capacity: torch.Tensor | None,
                               out: ChunkLayouts, stream=None) -> ChunkLayouts:
    _want(topk_idx, torch.int32, "topk_idx")
    if topk_idx.numel() < T * k or out.pos.numel() < T * k:
        raise ValueError("layout buffers smaller than T*k")
    if chunk_capacity is not None:
        _want(chunk_capacity, torch.int32, "chunk_capacity")
    n = ctypes.c_size_t(out.workspace.numel())
    _check("moe_dispatch_layout_chunks",
           load().moe_dispatch_layout_chunks(
               _ptr(topk_idx), T, out.chunk_tokens, E, k, R, int(capacity), _ptr(chunk_capacity),
               _ptr(out.expert_counts), _ptr(out.expert_offsets), _ptr(out.rank_counts),
               _ptr(out.rank_offsets), _ptr(out.pos), _ptr(out.row_src), _ptr(out.workspace),
               ctypes.byref(n), _stream(stream)))
    return out


def moe_route_layout_chunks(logits: torch.Tensor, k: int, R: int, capacity: int,
                            chunk_capacity: torch.Tensor | None, topk_idx: torch.Tensor,
                            topk_w: torch.Tensor, out: ChunkLayouts, stream=None) -> ChunkLayouts:
    """logits fp32 [T, E] -> topk_idx / topk_w [T, k] and every chunk's layout."""
    _want(logits, torch.float32, "logits")
    _want(topk_idx, torch.int32, "topk_idx")
    _want(topk_w, torch.float32, "topk_w")
    T, E = logits.shape
    if topk_idx.numel() < T * k or topk_w.numel() < T * k or out.pos.numel() < T * k:
        raise ValueError("route / layout buffers smaller than T*k")
    if chunk_capacity is not None:
        _want(chunk_capacity, torch.int32, "chunk_capacity")
    n = ctypes.c_size_t(out.workspace.numel())
    _check("moe_route_layout_chunks",
           load().moe_route_layout_chunks(
               _ptr(logits), T, out.chunk_tokens, E, k, R, int(capacity), _ptr(chunk_capacity),
               _ptr(topk_idx), _ptr(topk_w), _ptr(out.expert_counts), _ptr(out.expert_offsets),
               _ptr(out.rank_counts), _ptr(out.rank_offsets), _ptr(out.pos), _ptr(out.row_src),
               _ptr(out.workspace), ctypes.byref(n), _stream(stream)))
    return out


MOE_NOALLOC_SCRATCH_BYTES = 4 << 20  # static scratch of moe_route_layout_chunks_noalloc


def moe_route_layout_chunks_noalloc(logits: torch.Tensor, k: int, R: int, capacity: int,
                                    chunk_capacity: torch.Tensor | None, topk_idx: torch.Tensor,
                                    topk_w: torch.Tensor, out: ChunkLayouts,
                                    stream=None) -> ChunkLayouts:
    """As moe_route_layout_chunks, with the histogram scratch in the
    library's static device buffer: out.workspace is not used."""
    _want(logits, torch.float32, "logits")
    _want(topk_idx, torch.int32, "topk_idx")
    _want(topk_w, torch.float32, "topk_w")
    T, E = logits.shape
    if topk_idx.numel() < T * k or topk_w.numel() < T * k or out.pos.numel() < T * k:
        raise ValueError("route / layout buffers smaller than T*k")
    if chunk_capacity is not None:
        _want(chunk_capacity, torch.int32, "chunk_capacity")
    _check("moe_route_layout_chunks_noalloc",
           load().moe_route_layout_chunks_noalloc(
               _ptr(logits), T, out.chunk_tokens, E, k, R, int(capacity), _ptr(chunk_capacity),
               _ptr(topk_idx), _ptr(topk_w), _ptr(out.expert_counts), _ptr(out.expert_offsets),
               _ptr(out.rank_counts), _ptr(out.rank_offsets), _ptr(out.pos), _ptr(out.row_src),
               _stream(stream)))
    return out


def _want_scales(t: torch.Tensor | None, rows: int, quant: int, name: str):
    """A quantised row buffer's scale array: fp32, at least `rows` entries."""
    if quant == MOE_QUANT_BF16:
        return
    if t is None:
        raise ValueError(f"{name}: a quantised payload needs its fp32 scale array")
    _want(t, torch.float32, name)
    if t.numel() < rows:
        raise ValueError(f"{name} must hold {rows} scales")


def moe_dispatch_pack(x: torch.Tensor, T: int, H: int, k: int, pos: torch.Tensor, quant: int,
                      send: torch.Tensor, send_scales: torch.Tensor | None = None,
                      stream=None) -> None:
    """x bf16 [T, H] (or its int16/uint16 bits); send uint8 [rows, row_bytes];
    send_scales fp32 [rows] for the quantised formats.  quant may carry
    MOE_PACK_STREAM."""
    if x.element_size() != 2:
        raise ValueError("x must hold bf16 bits")
    _want(pos, torch.int32, "pos")
    if x.numel() < T * H or pos.numel() < T * k:
        raise ValueError("x / pos too small")
    _want_scales(send_scales, 0, quant & ~MOE_PACK_STREAM, "send_scales")
    _check("moe_dispatch_pack", load().moe_dispatch_pack(_ptr(x), T, H, k, _ptr(pos), quant,
                                                         _ptr(send), _ptr(send_scales),
                                                         _stream(stream)))


def moe_combine(recv: torch.Tensor, recv_scales: torch.Tensor | None, quant: int,
                pos: torch.Tensor, topk_w: torch.Tensor, T: int, H: int, k: int,
                out: torch.Tensor, stream=None) -> None:
    _want(pos, torch.int32, "pos")
    _want(topk_w, torch.float32, "topk_w")
    if out.element_size() != 2 or out.numel() < T * H:
        raise ValueError("out must hold T*H bf16 values")
    _want_scales(recv_scales, 0, quant, "recv_scales")
    _check("moe_combine", load().moe_combine(_ptr(recv), _ptr(recv_scales), quant, _ptr(pos),
                                             _ptr(topk_w), T, H, k, _ptr(out), _stream(stream)))


def moe_combine_pack(recv: torch.Tensor | None, recv_scales: torch.Tensor | None,
                     pos_c: torch.Tensor | None, topk_w: torch.Tensor | None, Tc: int,
                     out: torch.Tensor | None, x: torch.Tensor | None,
                     pos_p: torch.Tensor | None, Tp: int, send: torch.Tensor | None,
                     send_scales: torch.Tensor | None, H: int, k: int, quant: int,
                     stream=None) -> None:
    """moe_combine of Tc tokens and moe_dispatch_pack of Tp tokens in one
    launch; the tensors of a half with no tokens may be None (and the scale
    arrays are None for bf16).  quant may carry MOE_PACK_STREAM (pack half)."""
    fmt = quant & ~MOE_PACK_STREAM
    if Tc > 0:
        _want(pos_c, torch.int32, "pos_c")
        _want(topk_w, torch.float32, "topk_w")
        if out.element_size() != 2 or out.numel() < Tc * H:
            raise ValueError("out must hold Tc*H bf16 values")
        _want_scales(recv_scales, 0, fmt, "recv_scales")
    if Tp > 0:
        if x.element_size() != 2:
            raise ValueError("x must hold bf16 bits")
        _want(pos_p, torch.int32, "pos_p")
        if x.numel() < Tp * H or pos_p.numel() < Tp * k:
            raise ValueError("x / pos_p too small")
        _want_scales(send_scales, 0, fmt, "send_scales")
    _check("moe_combine_pack",
           load().moe_combine_pack(_ptr(recv), _ptr(recv_scales), _ptr(pos_c), _ptr(topk_w), Tc,
                                   _ptr(out), _ptr(x), _ptr(pos_p), Tp, _ptr(send),
                                   _ptr(send_scales), H, k, quant, _stream(stream)))


class RecvLayout(NamedTuple):
    recv_offsets: torch.Tensor   # [R, R+1] int32: segment starts per receiver (flat rows)
    group_offsets: torch.Tensor  # [E+1] int32: first grouped row per expert; [E] = N
    group_seg: torch.Tensor      # [E, R] int32: first grouped row of (expert, source)
    group_pos: torch.Tensor      # [max_rows] int32: grouped row of receive row q, -1 past N
    group_src: torch.Tensor      # [max_rows] int32: receive row of grouped row p, -1 past N

    @property
    def max_rows(self) -> int:
        return self.group_pos.numel()


def alloc_recv_layout(E: int, R: int, max_rows: int, device) -> RecvLayout:
    i32 = dict(dtype=torch.int32, device=device)
    return RecvLayout(torch.empty((R, R + 1), **i32), torch.empty(E + 1, **i32),
                      torch.empty((E, R), **i32), torch.empty(max(max_rows, 1), **i32)[:max_rows],
                      torch.empty(max(max_rows, 1), **i32)[:max_rows])


def _want_offsets(src_offsets: torch.Tensor, E: int, R: int):
    _want(src_offsets, torch.int32, "src_offsets")
    if src_offsets.numel() < R * (E + 1):
        raise ValueError("src_offsets must hold [R, E+1] int32")


def _want_rows(t: torch.Tensor, scales: torch.Tensor | None, rows: int, H: int, quant: int,
               name: str):
    if not t.is_contiguous() or t.numel() * t.element_size() < rows * moe_row_bytes(H, quant):
        raise ValueError(f"{name} must be contiguous and hold {rows} rows")
    _want_scales(scales, rows, quant, name + " scales")


def moe_recv_layout(src_offsets: torch.Tensor, E: int, R: int, out: RecvLayout,
                    stream=None) -> RecvLayout:
    _want_offsets(src_offsets, E, R)
    if (out.recv_offsets.numel() < R * (R + 1) or out.group_offsets.numel() < E + 1 or
            out.group_seg.numel() < E * R or out.group_src.numel() != out.max_rows):
        raise ValueError("RecvLayout buffers too small")
    _check("moe_recv_layout",
           load().moe_recv_layout(_ptr(src_offsets), E, R, out.max_rows, _ptr(out.recv_offsets),
                                  _ptr(out.group_offsets), _ptr(out.group_seg),
                                  _ptr(out.group_pos), _ptr(out.group_src), _stream(stream)))
    return out


def moe_recv_regroup(recv: torch.Tensor, recv_scales: torch.Tensor | None, max_rows: int,
                     H: int, quant: int, group_src: torch.Tensor, grouped: torch.Tensor,
                     grouped_scales: torch.Tensor | None, stream=None) -> None:
    _want(group_src, torch.int32, "group_src")
    if group_src.numel() < max_rows:
        raise ValueError("group_src shorter than max_rows")
    _want_rows(recv, recv_scales, max_rows, H, quant, "recv")
    _want_rows(grouped, grouped_scales, max_rows, H, quant, "grouped")
    _check("moe_recv_regroup",
           load().moe_recv_regroup(_ptr(recv), _ptr(recv_scales), max_rows, H, quant,
                                   _ptr(group_src), _ptr(grouped), _ptr(grouped_scales),
                                   _stream(stream)))


def moe_recv_ungroup(grouped: torch.Tensor, grouped_scales: torch.Tensor | None, max_rows: int,
                     H: int, quant: int, group_pos: torch.Tensor, recv: torch.Tensor,
                     recv_scales: torch.Tensor | None, stream=None) -> None:
    _want(group_pos, torch.int32, "group_pos")
    if group_pos.numel() < max_rows:
        raise ValueError("group_pos shorter than max_rows")
    _want_rows(recv, recv_scales, max_rows, H, quant, "recv")
    _want_rows(grouped, grouped_scales, max_rows, H, quant, "grouped")
    _check("moe_recv_ungroup",
           load().moe_recv_ungroup(_ptr(grouped), _ptr(grouped_scales), max_rows, H, quant,
                                   _ptr(group_pos), _ptr(recv), _ptr(recv_scales),
                                   _stream(stream)))
