"""Chunk driver: one MoE layer's dispatch/combine data path over HIP streams.

Follows the layer structure of the ThunderEP write-up (s3.3 pseudo-code, s2.1
and s2.2): route the whole batch once, then cut it into chunks (1/4..1/8 of the
batch is the recommended size), and for each chunk aggregate by destination
(layout + pack, optionally int8-compressed), exchange, run the experts and
combine.  Staging buffers are reused round-robin (the write-up's ring buffer)
instead of being allocated per chunk, and with two streams the dispatch of
chunk c overlaps the expert/combine work of chunk c-1, ordered only by
event record / stream-wait-event pairs (never a device or stream
synchronize inside the loop).

On one GPU the all-to-all is the identity: the receive buffer is the send
buffer.  ``standin=True`` runs the test expert y = x*(1+e/8) between dispatch
and combine (re-quantising on int8 return paths); otherwise combine reads the
send buffer directly (permute then unpermute).

All arithmetic happens in the HIP library; this module only allocates
buffers (torch), orders launches and passes pointers.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction
from math import ceil

import torch

from . import binding as B


def chunk_ranges(T: int, chunks: int):
    """Chunk c covers tokens [c*ceil(T/C), min(T, (c+1)*ceil(T/C)))."""
    step = -(-T // chunks) if T else 0
    return [(min(T, c * step), min(T, (c + 1) * step)) for c in range(chunks)]


def chunk_capacity(Tc: int, k: int, E: int, factor) -> int:
    """ceil(factor * Tc * k / E) in exact rational arithmetic; 0 = unlimited."""
    if not factor:
        return 0
    f = Fraction(factor).limit_denominator(1000)
    return int(ceil(f * Tc * k / E))


@dataclass
class Staging:
    layout: B.Layout
    send: torch.Tensor                 # uint8 [rows, stride]
    ret: torch.Tensor | None = None    # stand-in output (return buffer)
    ev_dispatched: torch.cuda.Event = field(default_factory=torch.cuda.Event)
    ev_combined: torch.cuda.Event = field(default_factory=torch.cuda.Event)
    used: bool = False


class KernelTimer:
    """Optional per-launch HIP events, recorded on the launch's own stream."""

    def __init__(self):
        self.spans: dict[str, list] = {}

    def start(self, name: str, stream):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        return (name, ev, stream)

    def stop(self, tok):
        name, ev0, stream = tok
        ev1 = torch.cuda.Event(enable_timing=True)
        ev1.record(stream)
        self.spans.setdefault(name, []).append((ev0, ev1))

    def ms(self) -> dict[str, list[float]]:
        return {n: [a.elapsed_time(b) for a, b in v] for n, v in self.spans.items()}

    def clear(self):
        self.spans.clear()


class DispatchCombine:
    """Preallocated buffers + launch order for one (T, H, E, k, R, chunks)."""

    def __init__(self, T: int, H: int, E: int, k: int, R: int, chunks: int = 1,
                 streams: int = 1, ring: int = 2, standin: bool = False, device="cuda"):
        if streams not in (1, 2):
            raise ValueError("streams must be 1 or 2")
        self.T, self.H, self.E, self.k, self.R = T, H, E, k, R
        self.chunks = chunks
        self.ranges = chunk_ranges(T, chunks)
        self.Tc = max((b - a for a, b in self.ranges), default=0)
        self.device = torch.device(device)
        self.standin = standin
        rows = max(self.Tc * k, 1)
        stride = max(B.moe_record_bytes(H, 0), B.moe_record_bytes(H, 1))
        self.idx = torch.empty((max(T, 1), k), dtype=torch.int32, device=self.device)
        self.w = torch.empty((max(T, 1), k), dtype=torch.float32, device=self.device)
        self.ring = [
            Staging(B.alloc_layout(self.Tc, E, k, R, self.device),
                    torch.empty((rows, stride), dtype=torch.uint8, device=self.device),
                    torch.empty((rows, stride), dtype=torch.uint8, device=self.device)
                    if standin else None)
            for _ in range(max(1, min(ring, chunks)))
        ]
        self.streams = streams
        if streams == 2:
            self.s_dispatch = torch.cuda.Stream(self.device)
            self.s_combine = torch.cuda.Stream(self.device)

    # ------------------------------------------------------------------
    def route(self, logits: torch.Tensor, stream=None):
        B.moe_route_topk(logits, self.k, self.idx, self.w, stream)

    def run(self, logits: torch.Tensor, x: torch.Tensor, out: torch.Tensor, quant: int = 0,
            capacity_factor=None, quant_ret: int | None = None, timer: KernelTimer | None = None):
        """One layer: route, then per chunk layout -> pack -> [stand-in] ->
        combine.  Asynchronous with respect to the host; `out` is ready when
        the caller's current stream reaches this point."""
        T, H, E, k, R = self.T, self.H, self.E, self.k, self.R
        if logits.shape != (T, E) or x.shape[0] != T or out.shape[0] != T:
            raise ValueError("logits/x/out shapes do not match the driver")
        quant_ret = quant if quant_ret is None else quant_ret
        cur = torch.cuda.current_stream(self.device)
        if self.streams == 2:
            sd, sc = self.s_dispatch, self.s_combine
            sd.wait_stream(cur)
            sc.wait_stream(cur)
        else:
            sd = sc = cur

        def timed(name, stream, fn):
            tok = timer.start(name, stream) if timer else None
            fn()
            if timer:
                timer.stop(tok)

        timed("route", sd, lambda: B.moe_route_topk(logits, k, self.idx, self.w, sd))
        for c, (t0, t1) in enumerate(self.ranges):
            st = self.ring[c % len(self.ring)]
            Tc = t1 - t0
            cap = chunk_capacity(Tc, k, E, capacity_factor)
            if self.streams == 2 and st.used:
                sd.wait_event(st.ev_combined)  # ring slot free again
            lay = st.layout
            idx_c = self.idx[t0:t1]
            timed("layout", sd, lambda: B.moe_dispatch_layout(idx_c, Tc, E, k, R, cap, lay, sd))
            timed("pack", sd, lambda: B.moe_dispatch_pack(x[t0:t1], Tc, H, k, lay.pos, quant,
                                                          st.send, sd))
            if self.streams == 2:
                st.ev_dispatched.record(sd)
                sc.wait_event(st.ev_dispatched)
            recv = st.send  # identity exchange
            if self.standin:
                ret = st.ret
                timed("standin", sc, lambda: B.moe_expert_standin(
                    recv, quant, lay.expert_offsets, E, max(Tc * k, 0), H, quant_ret, ret, sc))
                recv = ret
            timed("combine", sc, lambda: B.moe_combine(recv, quant_ret, lay.pos, self.w[t0:t1],
                                                       Tc, H, k, out[t0:t1], sc))
            if self.streams == 2:
                st.ev_combined.record(sc)
            st.used = True
        if self.streams == 2:
            cur.wait_stream(sd)
            cur.wait_stream(sc)

    def chunk_state(self, c: int) -> Staging:
        """Staging buffers of chunk c (valid while no later chunk reused them)."""
        return self.ring[c % len(self.ring)]


def run_stack(path: DispatchCombine, logits_per_layer, x: torch.Tensor, quants,
              capacity_factor=None, outs=None):
    """Layers chained as layer l+1 input = layer l output (no residual)."""
    cur = x
    outs = outs or [torch.empty_like(x) for _ in logits_per_layer]
    for l, (lg, q) in enumerate(zip(logits_per_layer, quants)):
        path.run(lg, cur, outs[l], quant=q, capacity_factor=capacity_factor)
        cur = outs[l]
    return outs
