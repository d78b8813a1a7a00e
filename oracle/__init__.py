"""CPU oracle for the MoE dispatch/combine data path -- TEST INFRASTRUCTURE.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
the two share no code: the arithmetic lives in ``oracle.c`` (plain C, built
with gcc into ``liboracle.so``) and this module only marshals numpy arrays.

Functions (each cites the passage it follows in ``oracle.c``):
  route_topk        O1  top-k + renormalised gate weights
  dispatch_layout   O2  histogram, scans, rank blocks, stable pos/row_src
  dispatch_pack     O3  bf16 copy or per-token int8 / int4 / fp8 record
  expert_standin    O5  test stand-in expert  y = x * (1 + e/8)
  combine           O6  gate-weighted sum back into token order
  roundtrip_token       O3+O6 for one token (identity exchange, no expert)
  run_layer             the chunk loop over O2..O6 for a whole layer
  recv_layout       O7  receiver block offsets and expert-major segments
  exchange          O8  the payload all-to-all as a block transpose
  regroup           O9  receive buffer -> per-expert contiguous rows (and back)
  run_ep_layer          O1..O9 with R source shards, all ranks on one device

Parity pins: every function above is pinned by ``tests/test_oracle_*.py``,
down to the last ulp of the fp32 gate weights (checked against the exact
value, evaluated in 60-digit decimal arithmetic and rounded once).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from fractions import Fraction
from math import ceil

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.oracle_route_topk.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_dispatch_layout.argtypes = [P, i64, i32, i32, i32, i64, P, P, P, P, P, P]
    lib.oracle_dispatch_pack.argtypes = [P, i64, i32, i32, P, i32, P]
    lib.oracle_expert_standin.argtypes = [P, i32, P, i32, i32, i32, P]
    lib.oracle_combine.argtypes = [P, i32, P, P, i64, i32, i32, P]
    lib.oracle_roundtrip_token.argtypes = [P, i32, i32, P, P, i32, P]
    lib.oracle_recv_layout.argtypes = [P, i32, i32, i64, P, P, P, P, P]
    lib.oracle_exchange.argtypes = [P, i64, P, i32, i32, i64, P, i32]
    lib.oracle_regroup.argtypes = [P, P, i32, i32, i64, P, i32]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_float
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_float_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_float_to_bf16.restype = ctypes.c_uint16
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_record_bytes.argtypes = [i32, i32]
    lib.oracle_record_bytes.restype = i64
    for name in ("oracle_route_topk", "oracle_dispatch_layout", "oracle_dispatch_pack",
                 "oracle_expert_standin", "oracle_combine", "oracle_roundtrip_token",
                 "oracle_recv_layout", "oracle_exchange", "oracle_regroup"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: precondition failed (rc={rc})")


def record_bytes(H: int, quant: int) -> int:
    """Row stride of the send buffer: 2H (bf16) or H+16 (int8 record)."""
    return int(_load().oracle_record_bytes(H, quant))


def float_to_bf16(v: float) -> int:
    return int(_load().oracle_float_to_bf16(float(v)))


def bf16_to_double(b: int) -> float:
    return float(_load().oracle_bf16_to_double(int(b)))


def floats_to_bf16(a: np.ndarray) -> np.ndarray:
    """Element-wise oracle RNE (slow; for small arrays in tests)."""
    lib = _load()
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    for i, v in enumerate(flat.tolist()):
        out[i] = lib.oracle_float_to_bf16(v)
    return out.reshape(np.shape(a))


def e4m3_decode(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for S.1111.111)."""
    return float(_load().oracle_e4m3_decode(int(code)))


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 code of a finite |v| <= 464, ties to even."""
    return int(_load().oracle_e4m3_encode(float(v)))


def route_topk(logits: np.ndarray, k: int):
    """O1.  logits fp32 [T, E] -> (idx int32 [T, k], w fp32 [T, k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    _check(_load().oracle_route_topk(_p(logits), T, E, k, _p(idx), _p(w)), "route_topk")
    return idx, w


@dataclass
class Layout:
    expert_counts: np.ndarray   # [E]   raw histogram
    expert_offsets: np.ndarray  # [E+1] exclusive scan of kept rows
    rank_counts: np.ndarray     # [R]
    rank_offsets: np.ndarray    # [R+1]
    pos: np.ndarray             # [Tc, k] row per slot, -1 = dropped
    row_src: np.ndarray         # [Tc*k] slot per row, -1 past N

    @property
    def n_rows(self) -> int:
        return int(self.expert_offsets[-1])


def dispatch_layout(idx: np.ndarray, E: int, R: int, capacity: int = 0) -> Layout:
    """O2 for one chunk.  idx int32 [Tc, k]; capacity <= 0 means unlimited."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Tc, k = idx.shape
    ec = np.empty(E, dtype=np.int32)
    eo = np.empty(E + 1, dtype=np.int32)
    rc = np.empty(R, dtype=np.int32)
    ro = np.empty(R + 1, dtype=np.int32)
    pos = np.empty((Tc, k), dtype=np.int32)
    row_src = np.empty(Tc * k, dtype=np.int32)
    _check(_load().oracle_dispatch_layout(_p(idx), Tc, E, k, R, int(capacity), _p(ec), _p(eo),
                                          _p(rc), _p(ro), _p(pos), _p(row_src)),
           "dispatch_layout")
    return Layout(ec, eo, rc, ro, pos, row_src)


def dispatch_pack(x_bits: np.ndarray, pos: np.ndarray, quant: int, n_rows: int | None = None,
                  fill: int = 0) -> np.ndarray:
    """O3 for one chunk.  x_bits uint16 [Tc, H] (bf16 bits) -> send uint8 [rows, stride]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    Tc, H = x_bits.shape
    k = pos.shape[1]
    rows = Tc * k if n_rows is None else n_rows
    send = np.full((rows, record_bytes(H, quant)), fill, dtype=np.uint8)
    _check(_load().oracle_dispatch_pack(_p(x_bits), Tc, H, k, _p(pos), quant, _p(send)),
           "dispatch_pack")
    return send


def expert_standin(recv: np.ndarray, quant_in: int, expert_offsets: np.ndarray, H: int,
                   quant_out: int) -> np.ndarray:
    """O5.  Returns a buffer of the same row count with stride for quant_out."""
    recv = np.ascontiguousarray(recv, dtype=np.uint8)
    eo = np.ascontiguousarray(expert_offsets, dtype=np.int32)
    E = eo.shape[0] - 1
    ret = np.zeros((recv.shape[0], record_bytes(H, quant_out)), dtype=np.uint8)
    _check(_load().oracle_expert_standin(_p(recv), quant_in, _p(eo), E, H, quant_out, _p(ret)),
           "expert_standin")
    return ret


def combine(ret: np.ndarray, quant: int, pos: np.ndarray, w: np.ndarray, H: int) -> np.ndarray:
    """O6 for one chunk -> out uint16 [Tc, H] (bf16 bits)."""
    ret = np.ascontiguousarray(ret, dtype=np.uint8)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    Tc, k = pos.shape
    out = np.empty((Tc, H), dtype=np.uint16)
    _check(_load().oracle_combine(_p(ret), quant, _p(pos), _p(w), Tc, H, k, _p(out)), "combine")
    return out


def roundtrip_token(xrow: np.ndarray, pos_t: np.ndarray, w_t: np.ndarray, quant: int) -> np.ndarray:
    """O3 then O6 for a single token (identity exchange, no expert)."""
    xrow = np.ascontiguousarray(xrow, dtype=np.uint16)
    pos_t = np.ascontiguousarray(pos_t, dtype=np.int32)
    w_t = np.ascontiguousarray(w_t, dtype=np.float32)
    H = xrow.shape[0]
    out = np.empty(H, dtype=np.uint16)
    _check(_load().oracle_roundtrip_token(_p(xrow), H, pos_t.shape[0], _p(pos_t), _p(w_t), quant,
                                          _p(out)), "roundtrip_token")
    return out


def chunk_bounds(T: int, chunks: int):
    """Chunk c covers tokens [c*ceil(T/C), min(T, (c+1)*ceil(T/C)))."""
    step = -(-T // chunks) if T else 0
    out = []
    for c in range(chunks):
        t0 = min(T, c * step)
        t1 = min(T, (c + 1) * step)
        out.append((t0, t1))
    return out


def capacity_for(Tc: int, k: int, E: int, factor) -> int:
    """Per-chunk expert capacity ceil(factor * Tc * k / E) in exact arithmetic
    ([Sparse] s2.1 capacity factor); factor None/0 -> 0 (unlimited)."""
    if not factor:
        return 0
    f = Fraction(factor).limit_denominator(1000)
    return int(ceil(f * Tc * k / E))


@dataclass
class LayerResult:
    idx: np.ndarray
    w: np.ndarray
    layouts: list
    sends: list
    rets: list
    out: np.ndarray


def run_layer(logits: np.ndarray, x_bits: np.ndarray, E: int, k: int, R: int, chunks: int = 1,
              quant: int = 0, capacity_factor=None, standin: bool = False,
              keep_buffers: bool = True, workers: int = 1) -> LayerResult:
    """One MoE layer's data path, chunk by chunk ([ThunderEP] s3.3 layer
    pseudo-code: route the whole batch, then per chunk aggregate, compress,
    exchange, run experts, combine).  The exchange is the identity; with
    ``standin`` the test expert y = x*(1+e/8) runs between dispatch and
    combine, re-quantising on int8 layers; without it combine reads the send
    buffer directly (permute-then-unpermute).  Chunks are independent; with
    ``workers`` > 1 they are evaluated by that many threads (the C calls
    release the GIL), each chunk still by the plain sequential code."""
    T, H = x_bits.shape
    idx, w = route_topk(logits, k)
    out = np.zeros((T, H), dtype=np.uint16)

    def one_chunk(bounds):
        t0, t1 = bounds
        Tc = t1 - t0
        cap = capacity_for(Tc, k, E, capacity_factor)
        lay = dispatch_layout(idx[t0:t1], E, R, cap)
        send = dispatch_pack(x_bits[t0:t1], lay.pos, quant, n_rows=max(lay.n_rows, 0))
        ret = expert_standin(send, quant, lay.expert_offsets, H, quant) if standin else send
        out[t0:t1] = combine(ret, quant, lay.pos, w[t0:t1], H)
        return lay, (send if keep_buffers else None), (ret if keep_buffers else None)

    bounds = chunk_bounds(T, chunks)
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            res = list(ex.map(one_chunk, bounds))
    else:
        res = [one_chunk(b) for b in bounds]
    layouts = [r[0] for r in res]
    sends = [r[1] for r in res] if keep_buffers else []
    rets = [r[2] for r in res] if keep_buffers else []
    return LayerResult(idx, w, layouts, sends, rets, out)


@dataclass
class RecvLayout:
    recv_offsets: np.ndarray   # [R, R+1] first row of source s's segment in receiver r's region
    group_offsets: np.ndarray  # [E+1]    first row of expert e in the grouped buffer
    group_seg: np.ndarray      # [E, R]   first row of source s's rows of expert e
    group_pos: np.ndarray      # [max_rows] grouped row of receive row q, -1 past N
    group_src: np.ndarray      # [max_rows] receive row of grouped row p, -1 past N

    @property
    def n_rows(self) -> int:
        return int(self.group_offsets[-1])


def recv_layout(src_offsets: np.ndarray, R: int, max_rows: int | None = None) -> RecvLayout:
    """O7.  src_offsets int32 [R, E+1]: every source's kept expert offsets.
    The row maps have max_rows entries (default: the total row count N)."""
    so = np.ascontiguousarray(src_offsets, dtype=np.int32)
    E = so.shape[1] - 1
    assert so.shape[0] == R
    if max_rows is None:
        max_rows = int(np.diff(so, axis=1).sum())
    ro = np.empty((R, R + 1), dtype=np.int32)
    go = np.empty(E + 1, dtype=np.int32)
    gs = np.empty((E, R), dtype=np.int32)
    gp = np.empty(max(max_rows, 1), dtype=np.int32)
    gsrc = np.empty(max(max_rows, 1), dtype=np.int32)
    _check(_load().oracle_recv_layout(_p(so), R, E, max_rows, _p(ro), _p(go), _p(gs), _p(gp),
                                      _p(gsrc)), "recv_layout")
    return RecvLayout(ro, go, gs, gp[:max_rows], gsrc[:max_rows])


def exchange(send: np.ndarray, source_rows: int, src_offsets: np.ndarray, R: int,
             recv: np.ndarray | None = None, reverse: bool = False) -> np.ndarray:
    """O8.  send uint8 [R*source_rows, stride] (source s at row s*source_rows).
    Forward: returns the flat receive buffer (same shape).  reverse: copies
    ``recv`` back into ``send`` (modified in place) and returns it."""
    so = np.ascontiguousarray(src_offsets, dtype=np.int32)
    E = so.shape[1] - 1
    assert send.flags["C_CONTIGUOUS"] and send.dtype == np.uint8
    if recv is None:
        recv = np.zeros_like(send)
    assert recv.flags["C_CONTIGUOUS"] and recv.shape[1] == send.shape[1]
    _check(_load().oracle_exchange(_p(send), source_rows, _p(so), R, E, send.shape[1], _p(recv),
                                   1 if reverse else 0), "exchange")
    return send if reverse else recv


def regroup(recv: np.ndarray, src_offsets: np.ndarray, R: int, grouped: np.ndarray | None = None,
            reverse: bool = False) -> np.ndarray:
    """O9.  Forward: flat receive buffer -> grouped buffer (returned).
    reverse: grouped -> receive order, written into ``recv`` and returned."""
    so = np.ascontiguousarray(src_offsets, dtype=np.int32)
    E = so.shape[1] - 1
    assert recv.flags["C_CONTIGUOUS"] and recv.dtype == np.uint8
    if grouped is None:
        grouped = np.zeros_like(recv)
    _check(_load().oracle_regroup(_p(recv), _p(so), R, E, recv.shape[1], _p(grouped),
                                  1 if reverse else 0), "regroup")
    return recv if reverse else grouped


@dataclass
class EPResult:
    idx: np.ndarray
    w: np.ndarray
    layouts: list          # per source (oracle Layout)
    rl: RecvLayout
    send: np.ndarray       # [R*source_rows, stride] all sources' send buffers
    recv: np.ndarray       # flat receive buffer
    grouped: np.ndarray    # per-expert contiguous rows
    out: np.ndarray


def run_ep_layer(logits: np.ndarray, x_bits: np.ndarray, E: int, k: int, R: int, quant: int = 0,
                 capacity_factor=None, standin: bool = True) -> EPResult:
    """One layer with the batch split into R consecutive source shards (rank
    s holds tokens [s*ceil(T/R), ...)), every rank simulated on one device:
    route, per-source layout and pack, exchange, regroup by expert, stand-in
    experts on the grouped rows, regroup back, return exchange, per-source
    combine ([Perseus] s1.1 four steps; [NCCL-EP] s3.3 flat buffers)."""
    T, H = x_bits.shape
    idx, w = route_topk(logits, k)
    bounds = chunk_bounds(T, R)
    source_rows = (bounds[0][1] - bounds[0][0]) * k if T else 0
    stride = record_bytes(H, quant)
    send = np.zeros((R * source_rows, stride), dtype=np.uint8)
    layouts = []
    for s, (t0, t1) in enumerate(bounds):
        cap = capacity_for(t1 - t0, k, E, capacity_factor)
        lay = dispatch_layout(idx[t0:t1], E, R, cap)
        layouts.append(lay)
        if t1 > t0:
            send[s * source_rows:(s + 1) * source_rows][:(t1 - t0) * k] = dispatch_pack(
                x_bits[t0:t1], lay.pos, quant)
    src_offsets = np.stack([lay.expert_offsets for lay in layouts])
    rl = recv_layout(src_offsets, R)
    recv = exchange(send, source_rows, src_offsets, R)
    grouped = regroup(recv, src_offsets, R)
    ret_g = expert_standin(grouped, quant, rl.group_offsets, H, quant) if standin else grouped
    ret_recv = regroup(np.zeros_like(recv), src_offsets, R, grouped=ret_g, reverse=True)
    ret_send = exchange(np.zeros_like(send), source_rows, src_offsets, R, recv=ret_recv,
                        reverse=True)
    out = np.zeros((T, H), dtype=np.uint16)
    for s, (t0, t1) in enumerate(bounds):
        if t1 > t0:
            out[t0:t1] = combine(ret_send[s * source_rows:(s + 1) * source_rows], quant,
                                 layouts[s].pos, w[t0:t1], H)
    return EPResult(idx, w, layouts, rl, send, recv, grouped, out)
