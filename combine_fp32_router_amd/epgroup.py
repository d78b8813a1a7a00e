"""All R ranks of one expert-parallel group on one device.

The batch is cut into R consecutive token shards, shard s playing source
rank s.  Each rank routes, lays out and packs its shard into its own flat
send buffer (one segment per destination rank, NCCL EP article s3.3); the
payload all-to-all becomes a block transpose into the ranks' receive
buffers (``moe_exchange_blocks``, a stand-in for the collective); each
receiver computes its row maps (``moe_recv_layout``) and regroups its rows
into one run per expert (``moe_recv_regroup``),
the experts run (the test stand-in y = x*(1+e/8)), the rows go back to
arrival order (``moe_recv_ungroup``) and through the reverse exchange, and
every source combines its own tokens (Perseus write-up s1.1: gate, dispatch,
experts, combine).

Every buffer holds all ranks end to end, so one launch of each kernel does
the work of all R ranks.  With capacity off, the grouped buffer equals the
single-source dispatch of the whole batch, and the output equals the
chunked layer's with one chunk per shard.  All arithmetic runs in the HIP
library; this module allocates (torch) and orders launches.
"""
from __future__ import annotations

import torch

from . import binding as B
from . import harness as HN
from .driver import KernelTimer, chunk_capacity, chunk_ranges


class EPGroup:
    def __init__(self, T: int, H: int, E: int, k: int, R: int, standin: bool = True,
                 device="cuda"):
        self.T, self.H, self.E, self.k, self.R = T, H, E, k, R
        self.device = torch.device(device)
        self.standin = standin
        self.bounds = chunk_ranges(T, R)
        self.Ts = max((b - a for a, b in self.bounds), default=0)
        self.source_rows = self.Ts * k
        self.max_rows = R * self.source_rows
        stride = max(B.moe_row_bytes(H, q) for q in (0, 1, 2, 3))
        rows = max(self.max_rows, 1)
        dev = self.device
        self.idx = torch.empty((max(T, 1), k), dtype=torch.int32, device=dev)
        self.w = torch.empty((max(T, 1), k), dtype=torch.float32, device=dev)
        self.lay = B.alloc_layout_chunks(T, max(self.Ts, 1), E, k, R, dev, R)
        # sources past the last token (T < R) have no layout launch: zero rows
        self.lay.expert_offsets.zero_()
        self.src_offsets = self.lay.expert_offsets[:R]
        self.views = [B.layout_view(self.lay, s, T) for s in range(R)]
        self.rl = B.alloc_recv_layout(E, R, self.max_rows, dev)
        self.send = torch.empty((rows, stride), dtype=torch.uint8, device=dev)
        self.recv = torch.empty_like(self.send)
        self.grouped = torch.empty_like(self.send)
        self.ret = torch.empty_like(self.send) if standin else None
        # one fp32 scale per row of each buffer (quantised payloads)
        scales = lambda: torch.empty(rows, dtype=torch.float32, device=dev)
        self.send_scales, self.recv_scales, self.grouped_scales = scales(), scales(), scales()
        self.ret_scales = scales() if standin else None
        self._caps = {}

    def _source_caps(self, factor):
        key = str(factor)
        if key not in self._caps:
            caps = [chunk_capacity(t1 - t0, self.k, self.E, factor) for t0, t1 in self.bounds]
            caps += [0] * (self.lay.expert_offsets.shape[0] - len(caps))
            self._caps[key] = torch.tensor(caps, dtype=torch.int32, device=self.device)
        return self._caps[key]

    def send_rows(self, s: int, quant: int) -> torch.Tensor:
        """Source s's send buffer: rows are dense rows of the payload's
        stride, whatever the tensor's own row shape."""
        n = self.source_rows * B.moe_row_bytes(self.H, quant)
        return self.send.view(-1)[s * n:(s + 1) * n]

    def send_scales_of(self, s: int) -> torch.Tensor:
        """Scales of source s's send rows."""
        return self.send_scales[s * self.source_rows:(s + 1) * self.source_rows]

    def run(self, logits: torch.Tensor, x: torch.Tensor, out: torch.Tensor, quant: int = 0,
            capacity_factor=None, timer: KernelTimer | None = None):
        T, H, E, k, R = self.T, self.H, self.E, self.k, self.R
        if logits.shape != (T, E) or x.shape[0] != T or out.shape[0] != T:
            raise ValueError("logits/x/out shapes do not match the group")
        st = torch.cuda.current_stream(self.device)
        M = self.max_rows

        def timed(name, fn):
            tok = timer.start(name, st) if timer else None
            fn()
            if timer:
                timer.stop(tok)

        timed("route", lambda: B.moe_route_topk(logits, k, self.idx, self.w, st))
        caps = self._source_caps(capacity_factor) if capacity_factor else None
        timed("layout", lambda: B.moe_dispatch_layout_chunks(self.idx, T, E, k, R, 0, caps,
                                                              self.lay, st))
        for s, (t0, t1) in enumerate(self.bounds):
            if t1 > t0:
                timed("pack", lambda: B.moe_dispatch_pack(x[t0:t1], t1 - t0, H, k,
                                                          self.views[s].pos, quant,
                                                          self.send_rows(s, quant),
                                                          self.send_scales_of(s), st))
        so = self.src_offsets
        timed("recv_layout", lambda: B.moe_recv_layout(so, E, R, self.rl, st))
        timed("exchange", lambda: HN.moe_exchange_blocks(
            self.send, self.send_scales, self.source_rows, self.recv, self.recv_scales, M, H,
            quant, so, E, R, self.rl, False, st))
        timed("regroup", lambda: B.moe_recv_regroup(
            self.recv, self.recv_scales, M, H, quant, self.rl.group_src, self.grouped,
            self.grouped_scales, st))
        ret, ret_scales = self.grouped, self.grouped_scales
        if self.standin:
            timed("standin", lambda: HN.moe_expert_standin(
                self.grouped, self.grouped_scales, quant, self.rl.group_offsets, E, M, H, quant,
                self.ret, self.ret_scales, st))
            ret, ret_scales = self.ret, self.ret_scales
        timed("ungroup", lambda: B.moe_recv_ungroup(ret, ret_scales, M, H, quant,
                                                    self.rl.group_pos, self.recv,
                                                    self.recv_scales, st))
        timed("exchange_back", lambda: HN.moe_exchange_blocks(
            self.send, self.send_scales, self.source_rows, self.recv, self.recv_scales, M, H,
            quant, so, E, R, self.rl, True, st))
        for s, (t0, t1) in enumerate(self.bounds):
            if t1 > t0:
                timed("combine", lambda: B.moe_combine(
                    self.send_rows(s, quant), self.send_scales_of(s), quant, self.views[s].pos,
                    self.w[t0:t1], t1 - t0, H, k, out[t0:t1], st))
        return out
