"""Chunk driver: one MoE layer's dispatch/combine data path over HIP streams.

Follows the layer structure of the ThunderEP write-up (s3.3 pseudo-code, s2.1
and s2.2): route the whole batch once, then cut it into chunks (1/4..1/8 of the
batch is the recommended size), and for each chunk aggregate by destination
(layout + pack, optionally int8-compressed), exchange, run the experts and
combine.  Cross-stream ordering uses event record / stream-wait-event pairs
only (never a device or stream synchronize inside the loop).

Modes:
  streams=1  everything on the caller's stream, in chunk order; staging
             buffers reused round-robin (the write-up's ring buffer).
  streams=2  a control stream routes and lays out chunks 1.. (one fused
             call) while the caller's stream routes chunk 0 alone and runs
             its pack, so only chunk 0's route and layout lie on the data
             stream's critical path; the data stream waits once, before the
             launch that packs chunk 1, for the control stream's layouts.
             The big kernels never overlap each other (two HBM-bound kernels
             at once only share the bandwidth).  Cross-stream waits are kept
             to one per call because each is slow (on MI355X a waiting
             stream idles about 6 us even on an event already complete, up
             to 9 when the event completes during the wait, and recording
             an event delays the recording stream by about 5 us); with no
             exchange to overlap on one GPU the mode stays a few percent
             slower than one stream.
  streams=3  route, layout and every pack on a side stream, combines on the
             caller's stream, the staging ring guarded by events (the shape
             an exchange would overlap with; on one GPU the two big kernels
             only share bandwidth).

``stream_stores=True`` writes the send rows with streaming stores that the
last-level cache does not keep (MOE_PACK_STREAM): for when nothing reads them
back from this GPU soon after the pack (rows that leave for other GPUs, or
that come back after other traffic).  The default keeps them in that cache,
where the merged launch's combine of the same chunk finds them on one GPU.

Routing and layout go through the fused call (the router counts experts per
token group while it picks them, so the layout's counting pass disappears)
unless ``fused=False``; both give identical outputs.

With streams=1 or 2, at least two staging buffers and one payload format in
both directions, chunk c's combine and chunk c+1's pack share one launch
(moe_combine_pack: the combine's blocks first, then the pack's), so the
step runs C+1 big launches instead of 2C and each boundary's tail is filled
by the next kernel's ramp-up; ``merge=False`` keeps them apart.  Outputs
are identical either way.

On one GPU the all-to-all is the identity: the receive buffer is the send
buffer.  ``standin=True`` runs the test expert y = x*(1+e/8) between dispatch
and combine (re-quantising on int8 return paths); otherwise combine reads the
send buffer directly (permute then unpermute).

All arithmetic happens in the HIP library; this module only allocates
buffers (torch), orders launches and passes pointers.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from math import ceil

import torch

from . import binding as B
from . import harness as HN
from .hipevent import Event


def chunk_ranges(T: int, chunks: int):
    """Chunk c covers tokens [c*ceil(T/C), min(T, (c+1)*ceil(T/C)))."""
    step = -(-T // chunks) if T else 0
    return [(min(T, c * step), min(T, (c + 1) * step)) for c in range(chunks)]


# MI355X last-level cache (AMD Infinity Cache), shared by all XCDs.
LLC_BYTES = 256 << 20


def fit_chunks(T: int, H: int, k: int, quant: int, choices=(4, 8)) -> int:
    """Fewest chunks, among the write-up's 1/4..1/8-of-the-batch sizes, whose
    per-chunk send buffer (ceil(T/C)*k rows and their scales) fits the
    last-level cache, so that pack's output is still cached when its
    consumer reads it; the largest choice when none fits."""
    stride = B.moe_row_bytes(H, quant) + (4 if quant else 0)
    for c in sorted(choices):
        if -(-T // c) * k * stride <= LLC_BYTES:
            return c
    return max(choices)


def resolve_chunks(wl, quant: int) -> int:
    """A workload's chunk count; 0 means fit_chunks for the payload."""
    return wl.chunks if wl.chunks else fit_chunks(wl.T, wl.H, wl.k, quant)


def chunk_capacity(Tc: int, k: int, E: int, factor) -> int:
    """ceil(factor * Tc * k / E) in exact rational arithmetic; 0 = unlimited."""
    if not factor:
        return 0
    f = Fraction(factor).limit_denominator(1000)
    return int(ceil(f * Tc * k / E))


@dataclass
class Staging:
    layout: B.Layout
    send: torch.Tensor                 # uint8, >= Tc*k rows of the widest format
    send_scales: torch.Tensor          # fp32 [Tc*k]: scales of quantised send rows
    ret: torch.Tensor | None = None    # stand-in output (return buffer)
    ret_scales: torch.Tensor | None = None


class KernelTimer:
    """Optional per-launch HIP timing events, recorded on the launch's own
    stream, from a pool created before use (creating events is a host call
    too slow for a timed loop).  Each record still costs the stream a few
    microseconds, so timed wall-clock runs leave the timer off."""

    def __init__(self, names=None, pool: int = 0):
        self.names = set(names) if names else None
        self.tag = None  # spans are keyed name, or name@tag when a tag is set
        self.spans: dict[str, list] = {}
        self._pool = [Event(timing=True) for _ in range(pool)]

    def _event(self) -> Event:
        return self._pool.pop() if self._pool else Event(timing=True)

    def start(self, name: str, stream):
        if self.names is not None and name not in self.names:
            return None
        ev = self._event()
        ev.record(stream)
        return (f"{name}@{self.tag}" if self.tag else name, ev, stream)

    def stop(self, tok):
        if tok is None:
            return
        name, ev0, stream = tok
        ev1 = self._event()
        ev1.record(stream)
        self.spans.setdefault(name, []).append((ev0, ev1))

    def ms(self) -> dict[str, list[float]]:
        return {n: [a.elapsed_ms(b) for a, b in v] for n, v in self.spans.items()}


class DispatchCombine:
    """Preallocated buffers + launch order for one (T, H, E, k, R, chunks)."""

    def __init__(self, T: int, H: int, E: int, k: int, R: int, chunks: int = 1,
                 streams: int = 1, ring: int = 2, standin: bool = False, device="cuda",
                 fused: bool = True, merge: bool = True, stream_stores: bool = False):
        if streams not in (1, 2, 3):
            raise ValueError("streams must be 1, 2 or 3")
        self.T, self.H, self.E, self.k, self.R = T, H, E, k, R
        self.chunks = chunks
        self.ranges = chunk_ranges(T, chunks)
        self.Tc = max((b - a for a, b in self.ranges), default=0)
        self.device = torch.device(device)
        self.standin = standin
        self.streams = streams
        self.fused = fused  # route fused with the layout's counting pass
        # combine of chunk c and pack of chunk c+1 in one launch (one stream,
        # at least two staging buffers, one payload format both ways)
        self.merge = merge
        # send rows written with streaming stores (not kept in the last-level
        # cache): for when their consumer does not read them back soon
        self.pack_flags = B.MOE_PACK_STREAM if stream_stores else 0
        rows = max(self.Tc * k, 1)
        stride = max(B.moe_row_bytes(H, q) for q in (0, 1, 2, 3))
        self.idx = torch.empty((max(T, 1), k), dtype=torch.int32, device=self.device)
        self.w = torch.empty((max(T, 1), k), dtype=torch.float32, device=self.device)

        def buf():
            return (torch.empty((rows, stride), dtype=torch.uint8, device=self.device),
                    torch.empty(rows, dtype=torch.float32, device=self.device))

        # every chunk's layout lives in one batched allocation; staging
        # buffers are reused round-robin (pack and combine of a chunk are
        # ordered on one stream, so even a single buffer would be safe)
        self.lay = B.alloc_layout_chunks(T, max(self.Tc, 1), E, k, R, self.device, chunks)
        self.views = [B.layout_view(self.lay, c, T) for c in range(chunks)]
        nbuf = max(1, min(ring, chunks))
        self.nbuf = nbuf
        bufs = [(*buf(), *(buf() if standin else (None, None))) for _ in range(nbuf)]
        self.ring = [Staging(self.views[c], *bufs[c % nbuf]) for c in range(chunks)]
        self._caps = {}
        if streams in (2, 3):
            self.s_ctrl = torch.cuda.Stream(self.device)  # default priority on purpose
            self.ev_in = Event()
        if streams == 2:
            # chunk 0 is routed and laid out on the caller's stream while the
            # control stream does the other chunks: its own workspace
            t0, t1 = self.ranges[0]
            ws0 = max(B.route_layout_workspace_bytes(t1 - t0, max(self.Tc, 1), E, k, R),
                      B.layout_workspace_bytes(t1 - t0, E, k, R))
            ws0 = torch.empty(ws0, dtype=torch.uint8, device=self.device)
            self.lay0 = self.lay._replace(workspace=ws0)
            self.view0 = self.views[0]._replace(workspace=ws0)
            self.ev_rest = Event()  # chunks 1.. routed and laid out
        if streams == 3:
            self.ev_packed = [Event() for _ in range(chunks)]
            self.ev_combined = [Event() for _ in range(chunks)]
            self.ev_done = Event()

    def _chunk_caps(self, factor):
        """Device array of per-chunk capacities (cached per factor)."""
        key = str(factor)
        if key not in self._caps:
            caps = [chunk_capacity(t1 - t0, self.k, self.E, factor) for t0, t1 in self.ranges]
            self._caps[key] = torch.tensor(caps, dtype=torch.int32, device=self.device)
        return self._caps[key]

    def run(self, logits: torch.Tensor, x: torch.Tensor, out: torch.Tensor, quant: int = 0,
            capacity_factor=None, quant_ret: int | None = None, timer: KernelTimer | None = None):
        """One layer: route, then per chunk layout -> pack -> [stand-in] ->
        combine.  Asynchronous with respect to the host; `out` is ready when
        the caller's current stream reaches this point."""
        T, H, E, k, R = self.T, self.H, self.E, self.k, self.R
        if logits.shape != (T, E) or x.shape[0] != T or out.shape[0] != T:
            raise ValueError("logits/x/out shapes do not match the driver")
        quant_ret = quant if quant_ret is None else quant_ret
        data = torch.cuda.current_stream(self.device)
        ctrl = self.s_ctrl if self.streams in (2, 3) else data

        def timed(name, stream, fn):
            tok = timer.start(name, stream) if timer else None
            fn()
            if timer:
                timer.stop(tok)

        def pack(c):
            t0, t1 = self.ranges[c]
            st = self.ring[c]
            timed("pack", data, lambda: B.moe_dispatch_pack(
                x[t0:t1], t1 - t0, H, k, st.layout.pos, quant | self.pack_flags, st.send,
                st.send_scales, data))

        def returned(c):
            """Rows combine reads for chunk c (identity exchange): the send
            buffer, or the stand-in expert's output written from it now."""
            t0, t1 = self.ranges[c]
            st = self.ring[c]
            if not self.standin:
                return st.send, st.send_scales
            timed("standin", data, lambda: HN.moe_expert_standin(
                st.send, st.send_scales, quant, st.layout.expert_offsets, E,
                max((t1 - t0) * k, 0), H, quant_ret, st.ret, st.ret_scales, data))
            return st.ret, st.ret_scales

        def combine(c, recv):
            t0, t1 = self.ranges[c]
            timed("combine", data, lambda: B.moe_combine(
                recv[0], recv[1], quant_ret, self.ring[c].layout.pos, self.w[t0:t1], t1 - t0, H,
                k, out[t0:t1], data))

        def combine_pack(c, recv):
            t0, t1 = self.ranges[c]
            n0, n1 = self.ranges[c + 1]
            nxt = self.ring[c + 1]
            timed("combine_pack", data, lambda: B.moe_combine_pack(
                recv[0], recv[1], self.ring[c].layout.pos, self.w[t0:t1], t1 - t0, out[t0:t1],
                x[n0:n1], nxt.layout.pos, n1 - n0, nxt.send, nxt.send_scales, H, k,
                quant | self.pack_flags, data))

        def data_chunks(before_pack=lambda c: None):
            """pack -> [stand-in] -> combine for every chunk, in chunk order;
            merged, chunk c's combine and chunk c+1's pack share a launch."""
            merge = self.merge and self.nbuf >= 2 and quant_ret == quant and self.chunks >= 2
            if not merge:
                for c in range(self.chunks):
                    before_pack(c)
                    pack(c)
                    combine(c, returned(c))
                return
            before_pack(0)
            pack(0)
            recv = returned(0)
            for c in range(self.chunks - 1):
                before_pack(c + 1)
                combine_pack(c, recv)
                recv = returned(c + 1)
            combine(self.chunks - 1, recv)

        def route_and_layout(stream):
            """Route the whole batch and lay out every chunk: one fused call
            (two launches), or route then the batched layout."""
            caps = self._chunk_caps(capacity_factor) if capacity_factor else None
            if self.fused:
                timed("route_layout", stream, lambda: B.moe_route_layout_chunks(
                    logits, k, R, 0, caps, self.idx, self.w, self.lay, stream))
                return
            timed("route", stream, lambda: B.moe_route_topk(logits, k, self.idx, self.w, stream))
            timed("layout", stream, lambda: B.moe_dispatch_layout_chunks(
                self.idx, T, E, k, R, 0, caps, self.lay, stream))

        if self.streams == 2:
            # The control stream waits for everything the caller queued
            # before this call (the logits; earlier layers still reading idx,
            # w and the layouts), then routes and lays out chunks 1.. in one
            # fused call.  Meanwhile the caller's stream routes and lays out
            # chunk 0 (its own workspace) and packs it; it waits for the
            # control stream only before the launch that packs chunk 1.
            # Control work is enqueued first, so it starts as early as it can.
            t0, t1 = self.ranges[0]
            caps = self._chunk_caps(capacity_factor) if capacity_factor else None
            tail = self.chunks > 1 and t1 < T
            if tail:
                self.ev_in.record(data)
                self.ev_in.wait(ctrl)
                rest = B.layout_chunks_from(self.lay, 1)
                rcaps = None if caps is None else caps[1:]
                if self.fused:
                    timed("route_layout", ctrl, lambda: B.moe_route_layout_chunks(
                        logits[t1:], k, R, 0, rcaps, self.idx[t1:], self.w[t1:], rest, ctrl))
                else:
                    timed("route", ctrl, lambda: B.moe_route_topk(
                        logits[t1:], k, self.idx[t1:], self.w[t1:], ctrl))
                    timed("layout", ctrl, lambda: B.moe_dispatch_layout_chunks(
                        self.idx[t1:], T - t1, E, k, R, 0, rcaps, rest, ctrl))
                self.ev_rest.record(ctrl)
            if self.fused:
                timed("route_layout", data, lambda: B.moe_route_layout_chunks(
                    logits[t0:t1], k, R, 0, None if caps is None else caps[:1],
                    self.idx[t0:t1], self.w[t0:t1], self.lay0, data))
            else:
                cap0 = chunk_capacity(t1 - t0, k, E, capacity_factor)
                timed("route", data, lambda: B.moe_route_topk(
                    logits[t0:t1], k, self.idx[t0:t1], self.w[t0:t1], data))
                timed("layout", data, lambda: B.moe_dispatch_layout(
                    self.idx[t0:t1], t1 - t0, E, k, R, cap0, self.view0, data))

            def wait_layout(c):
                if c == 1 and tail:
                    self.ev_rest.wait(data)

            data_chunks(wait_layout)
        elif self.streams == 3:
            # Pack on the second stream, combine on the caller's: pack of
            # chunk c+1 (into the other staging buffer) runs while chunk c
            # combines, so each big kernel's ramp-up and tail overlap the
            # other's.  Waits: combine c after pack c; pack c+ring after
            # combine c (buffer reuse); none of them on an idle stream.
            pk = ctrl
            self.ev_in.record(data)
            self.ev_in.wait(pk)
            route_and_layout(pk)
            nbuf = len({id(st.send) for st in self.ring})

            def side_pack(c):
                t0, t1 = self.ranges[c]
                st = self.ring[c]
                if c >= nbuf:  # staging buffer reused: combine c-nbuf must be done
                    self.ev_combined[c - nbuf].wait(pk)
                timed("pack", pk, lambda: B.moe_dispatch_pack(
                    x[t0:t1], t1 - t0, H, k, st.layout.pos, quant | self.pack_flags, st.send,
                    st.send_scales, pk))
                self.ev_packed[c].record(pk)

            def main_combine(c):
                t0, t1 = self.ranges[c]
                st = self.ring[c]
                self.ev_packed[c].wait(data)
                recv, rscales = st.send, st.send_scales
                if self.standin:
                    timed("standin", data, lambda: HN.moe_expert_standin(
                        st.send, st.send_scales, quant, st.layout.expert_offsets, E,
                        max((t1 - t0) * k, 0), H, quant_ret, st.ret, st.ret_scales, data))
                    recv, rscales = st.ret, st.ret_scales
                timed("combine", data, lambda: B.moe_combine(
                    recv, rscales, quant_ret, st.layout.pos, self.w[t0:t1], t1 - t0, H, k,
                    out[t0:t1], data))
                self.ev_combined[c].record(data)

            # host order matters: a stream waits only for an event recorded
            # before the wait was issued, so combine c-nbuf is enqueued (and
            # its event recorded) before pack c, which waits on it
            for c in range(self.chunks):
                side_pack(c)
                if c - nbuf + 1 >= 0:
                    main_combine(c - nbuf + 1)
            for c in range(max(0, self.chunks - nbuf + 1), self.chunks):
                main_combine(c)
        else:
            # one route and one batched layout for all chunks, then the data
            route_and_layout(data)
            data_chunks()

    def chunk_state(self, c: int) -> Staging:
        """Staging buffers of chunk c (valid while no later chunk reused them;
        with streams=2 the send/return buffers hold the last chunk's rows)."""
        return self.ring[c % len(self.ring)]


def capture(fn, device="cuda", warmup: int = 2) -> torch.cuda.CUDAGraph:
    """Record fn() -- DispatchCombine.run calls with streams=1 or 2 -- as one
    HIP graph; graph.replay() then re-issues every launch with the same
    device addresses, reading whatever those buffers hold at replay time.
    fn runs `warmup` times on a side stream first (first calls cache device
    tables, such as per-chunk capacities, whose upload cannot be captured).
    The path issues no memset or host synchronisation.  With one stream the
    graph holds only kernel nodes; with two, the control stream forks from
    the caller's stream on an event and joins back through the event of
    its layouts, so its event waits become graph edges."""
    dev = torch.device(device)
    side = torch.cuda.Stream(dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph
