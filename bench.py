"""Benchmark of the single-GPU MoE dispatch+combine data path.

One step = one MoE layer's whole data path over one batch: route the batch
(fp32 top-k + renormalised gates), then for every chunk dispatch layout,
dispatch pack, identity exchange (the receive buffer is the send buffer) and
combine.  Inputs are resident in HBM before the timed region starts.

Default workload: T=16384 tokens, H=7168, E=256 experts, top-8, R=32
destination ranks, bf16 payload, Zipf(1.1)-skewed routing and 1% outlier rows
(x50), in 8 chunks: the fewest of the write-up's 1/4..1/8-batch chunk sizes
whose send buffer (235 MB) fits the 256 MB last-level cache.  The int8, int4
and fp8 payload variants of the same workload (4 chunks by the same rule)
are measured in the same run and reported under "variants".

value = algorithmic dispatch+combine bytes per step / wall time per step
(GB/s, 1e9 bytes), over the whole pipeline as it runs: combine reads much of
its chunk's send buffer from the last-level cache, where pack left it.
"hbm_cold" is the HBM-only figure: the same pipeline with the exchange a
one-step delay line (combine of chunk c reads the rows packed for chunk c in
the previous step, long evicted from that cache) and the pack's rows written
with streaming stores (MOE_PACK_STREAM), wall clock per step.
Its "kernels_swept" times pack and combine launched alone after a 1 GiB
cached read sweep (untimed) that leaves the cache holding only clean,
unrelated lines.  Algorithmic bytes per layer
(N = kept rows, S = bytes a row carries: 2H for bf16, H codes + a 4-byte
scale for int8 and fp8, H/2 + 4 for int4):
  route    T*E*4 + T*k*8
  layout   T*k*4 + 2*T*k*4
  pack     T*H*2 + T*k*4 + N*S
  combine  N*S + T*k*8 + T*H*2
The 2*N*S part is the 2*T*k*H*b exchange volume of the communication-wall
explainer.  "copy_peak" is a plain copy of 4 GiB measured in the same run
(the achievable rate for a read+write stream, against which the path's
rates are also given).

"configs" measures the other workloads (one-chunk mid shape, the dsv3 shape
at 4 chunks, the 4-layer qwen3-like stack on one and two streams, the large
shape) with fewer steps.  The CPU leg times the oracle (plain C) on the
same work, single-threaded and on all host cores, and compares the GPU's
results on a sampled chunk of every payload with the oracle's ("parity").

Prints one JSON line.  Also: --json-out FILE writes the same line to a file.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s & % of peak at T=16384,H=7168,E=256,k=8"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
FLUSH_BYTES = 1 << 30  # read sweep that evicts the 256 MB last-level cache
_CSRC = "combine_fp32_router_amd/csrc/"
# every file a kernel is compiled from: committed traffic counters stay valid
# only while all of them are unchanged
KERNEL_SOURCES = {
    "pack": [_CSRC + f for f in ("dispatch_pack.hip", "pack_rows.hpp", "common.hpp")],
    "combine": [_CSRC + f for f in ("combine.hip", "combine_rows.hpp", "common.hpp")],
    "combine_pack": [_CSRC + f for f in ("combine_pack.hip", "combine_rows.hpp",
                                         "pack_rows.hpp", "common.hpp")],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--chunks", type=int, default=0, help="0 = the workload's own")
    ap.add_argument("--quant", type=int, default=None,
                    help="primary payload of one-layer workloads: 0 bf16, 1 int8, 2 int4, 3 fp8 "
                         "(default: the workload's own)")
    ap.add_argument("--streams", type=int, default=0, choices=(0, 1, 2, 3),
                    help="0: the workload's own; 2: route+layout run ahead on a control "
                         "stream; 3: pack and combine on separate streams")
    ap.add_argument("--no-variant", action="store_true", help="skip the other payloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the all-cores oracle leg (0: the host's CPU share, <= 16)")
    ap.add_argument("--no-kernel-events", action="store_true")
    ap.add_argument("--ring", type=int, default=2,
                    help="staging buffers reused across chunks (1: one buffer, safe on one stream)")
    ap.add_argument("--unfused", action="store_true",
                    help="route and layout as separate calls (three launches, not two)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as one HIP graph (one stream)")
    ap.add_argument("--no-merge", action="store_true",
                    help="pack and combine of every chunk as separate launches (2C big "
                         "launches instead of C+1)")
    ap.add_argument("--stream-stores", action="store_true",
                    help="pipeline with streaming send-row stores (MOE_PACK_STREAM)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-cold (HBM-only) leg")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the dispatch/combine + concurrent GEMM measurement")
    ap.add_argument("--no-ep", action="store_true",
                    help="skip the receiver-side (all ranks on one device) measurement")
    ap.add_argument("--json-out", default="")
    ap.add_argument("--copy-probe", type=float, default=0.0,
                    help="only run the copy and read probes over this many GiB and exit")
    return ap.parse_args()


PAYLOADS = ("bf16", "int8", "int4", "fp8")


def payload_bytes(H, quant):
    """Bytes one send row carries: 2H (bf16); H (int8, fp8) or H/2 (int4)
    codes plus the row's 4-byte scale, which travels in its own array."""
    return (2 * H, H + 4, H // 2 + 4, H + 4)[quant]


def algorithmic_bytes(T, H, E, k, N, quant):
    S = payload_bytes(H, quant)
    route = T * E * 4 + T * k * 8
    layout = T * k * 4 + 2 * T * k * 4
    pack = T * H * 2 + T * k * 4 + N * S
    comb = N * S + T * k * 8 + T * H * 2
    # a merged launch combines one chunk and packs the next: for chunks of
    # the same shape, one chunk's pack + combine bytes
    return dict(route=route, layout=layout, route_layout=route + layout, pack=pack,
                combine=comb, combine_pack=pack + comb, total=route + layout + pack + comb)


def source_sha(paths):
    """First 16 hex digits of sha256 over the files' bytes, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, quant):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, valid
    only while the kernel source is unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_{PAYLOADS[quant]}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return d


def chunk_bounds(T, chunks):
    step = -(-T // chunks)
    return [(min(T, c * step), min(T, (c + 1) * step)) for c in range(chunks)]


def step_bytes(wl, quants, chunks, kept):
    """Algorithmic bytes of one step, summed over layers and chunks."""
    tot = 0
    for q, kl in zip(quants, kept):
        for c, (t0, t1) in enumerate(chunk_bounds(wl.T, chunks)):
            tot += algorithmic_bytes(t1 - t0, wl.H, wl.E, wl.k, kl[c], q)["total"]
    return tot


def weights_max_rel_err(w, w_ref):
    """Largest |w - ref| / |ref| over the gate weights; a weight the
    reference gives as 0 (underflow) must be 0 too (else inf); NaN -> inf."""
    g, r = np.asarray(w, np.float64), np.asarray(w_ref, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(r == 0, np.where(g == 0, 0.0, np.inf), np.abs(g - r) / np.abs(r))
    return float(np.max(np.where(np.isnan(rel), np.inf, rel), initial=0.0))


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ probes
DST_SHIFT = 4096


def probe_peaks(torch, nbytes=4 << 30, reps=10, warmup=3):
    """Copy of nbytes (read + write traffic 2*nbytes) and a streaming read of
    nbytes, timed with HIP events: the achievable rates the path is
    compared with."""
    from combine_fp32_router_amd import harness as HN
    from combine_fp32_router_amd.hipevent import Event

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
    # the destination 4 KiB past the allocation's start: with both buffers at
    # the same offset modulo 64 KiB the copy measured 1% slower
    dst_buf = torch.empty(nbytes + DST_SHIFT, dtype=torch.uint8, device="cuda")
    dst = dst_buf[DST_SHIFT:]
    res = {"bytes": nbytes}
    for name, mode, traffic in (("copy", HN.MOE_PROBE_COPY, 2 * nbytes),
                                ("read", HN.MOE_PROBE_READ_STREAM, nbytes)):
        if mode != HN.MOE_PROBE_COPY:
            dst[:4].zero_()
        for _ in range(warmup):
            HN.moe_stream_probe(src, dst, nbytes, mode)
        evs = [(Event(timing=True), Event(timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()
            HN.moe_stream_probe(src, dst, nbytes, mode)
            b.record()
        torch.cuda.synchronize()
        ms = [a.elapsed_ms(b) for a, b in evs]
        res[f"{name}_gbs"] = round(traffic / (np.mean(ms) * 1e-3) / 1e9, 1)
        res[f"{name}_gbs_best"] = round(traffic / (min(ms) * 1e-3) / 1e9, 1)
        res[f"{name}_avg_us"] = round(1e3 * float(np.mean(ms)), 2)
        if mode == HN.MOE_PROBE_COPY:  # before the read sweep writes its digests into dst
            assert torch.equal(src[:1 << 20], dst[:1 << 20])
            assert torch.equal(src[-(1 << 20):], dst[-(1 << 20):])
    assert int(dst[:4].view(torch.int32).item()) == 0  # no all-ones vector in src
    res["note"] = ("moe_stream_probe: copy = 4 KiB tiles, streaming loads, streaming "
                   "device-scope stores, destination 4 KiB off the source's 64 KiB alignment; "
                   f"read = 16 KiB tiles, streaming loads; HIP-event average over {reps} launches")
    del src, dst, dst_buf
    torch.cuda.empty_cache()
    log(f"copy peak {res['copy_gbs']} GB/s, read {res['read_gbs']} GB/s over {nbytes >> 30} GiB")
    return res


class Flush:
    """A cached read sweep of 1 GiB: evicts the last-level cache and leaves it
    holding only clean lines of this buffer."""

    def __init__(self, torch):
        from combine_fp32_router_amd import harness as HN
        self.HN = HN
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda").fill_(5)
        self.count = torch.zeros(1, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.HN.moe_stream_probe(self.buf, self.count, FLUSH_BYTES, self.HN.MOE_PROBE_READ_CACHED)


# ------------------------------------------------------------------ GPU legs
class Inputs:
    """Two device copies of a workload's inputs (hidden rows and every
    layer's logits); step s reads copy s % 2.  In a model a layer's input is
    new at every call, so no timed step may find the previous step's inputs
    in the 256 MB last-level cache: re-reading one copy every step, the
    delay-line pipeline (whose other traffic does not allocate in that cache)
    ran 10-11% faster than with two copies (T=16384, H=7168 bf16 0.717 against
    0.788 ms, int8 0.394 against 0.440), the ordinary pipeline ~0.5%."""

    def __init__(self, x_d, logits_list):
        self.x = [x_d, x_d.clone()]
        self.logits = [list(logits_list), [lg.clone() for lg in logits_list]]

    def __call__(self, s):
        return self.x[s % 2], self.logits[s % 2]


def run_step(path, logits_list, x_d, outs, quants, cf, timer=None):
    """One step: every layer of the workload, layer l+1 reading layer l's
    output (ping-pong output buffers)."""
    cur = x_d
    for l, (lg, q) in enumerate(zip(logits_list, quants)):
        if timer is not None:
            timer.tag = f"L{l}" if len(quants) > 1 else None
        out = outs[l % 2]
        path.run(lg, cur, out, quant=q, capacity_factor=cf, timer=timer)
        cur = out
    return cur


def measure(args, wl, quants, chunks, streams, inp, outs, torch, D, steps, warmup,
            kernel_events=True):
    """Warm up, then time exactly `steps` steps with nothing else on the
    stream (wall clock + one event pair around the whole region); step i
    reads input copy i % 2 (Inputs).  Then run the same number of steps again
    with HIP events around every launch, on the launch's own stream, for the
    per-kernel durations: a recorded event delays the next kernel by several
    microseconds, so per-kernel events stay out of the wall-clock region.
    Returns the kept rows of every layer's chunks (read after the timed
    region) and the driver."""
    from combine_fp32_router_amd.hipevent import Event

    cf = wl.capacity_factor
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=chunks, streams=streams,
                             ring=args.ring, fused=not args.unfused, merge=not args.no_merge,
                             stream_stores=getattr(args, "stream_stores", False))

    def eager(i, timer=None):
        x, lgs = inp(i)
        run_step(path, lgs, x, outs, quants, cf, timer=timer)

    step = eager
    if args.graph:
        if streams == 3:
            raise SystemExit("--graph captures the one- and two-stream paths")
        graphs = [D.capture(lambda: eager(0)), D.capture(lambda: eager(1))]
        step = lambda i: graphs[i % 2].replay()  # noqa: E731
    i = 0
    for _ in range(warmup):
        step(i)
        i += 1
    ev0, ev1 = Event(timing=True), Event(timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step(i)
        i += 1
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    gpu_ms = ev0.elapsed_ms(ev1) / steps
    kms = {}
    if kernel_events:
        launches = len(quants) * (2 + 3 * chunks)
        timer = D.KernelTimer(pool=2 * launches * steps)
        torch.cuda.synchronize()
        for _ in range(steps):
            eager(i, timer=timer)
            i += 1
        torch.cuda.synchronize()
        kms = timer.ms()
    # kept rows per layer and chunk (capacity may drop some): one more step,
    # layer by layer, reading each layer's expert offsets
    kept = []
    cur, lgs = inp(i)
    for l, (lg, q) in enumerate(zip(lgs, quants)):
        path.run(lg, cur, outs[l % 2], quant=q, capacity_factor=cf)
        cur = outs[l % 2]
        torch.cuda.synchronize()
        kept.append([int(path.views[c].expert_offsets[-1].item()) for c in range(chunks)])
    return wall_ms, gpu_ms, kms, kept, path


def kernel_report(kms, wl, quants, chunks, steps, kept):
    """Average (and median, minimum) launch duration and achieved GB/s per
    kernel: algorithmic bytes of one launch / its average HIP-event duration.
    Keys are the kernel name, or name@L<layer> for multi-layer steps."""
    rep = {}
    Tc = -(-wl.T // chunks)
    for key, spans in kms.items():
        if not spans:
            continue
        name, _, tag = key.partition("@")
        layer = int(tag[1:]) if tag else 0
        q = quants[layer]
        avg = float(np.mean(spans))
        per_step = len(spans) / steps
        if name in ("route", "layout", "route_layout"):  # per layer-step (or chunk 0 / rest)
            b = int(algorithmic_bytes(wl.T, wl.H, wl.E, wl.k, wl.T * wl.k, q)[name] / per_step)
        else:  # per chunk: the average chunk's bytes
            n_avg = sum(kept[layer]) / chunks
            b = int(algorithmic_bytes(Tc, wl.H, wl.E, wl.k, n_avg, q)[name])
        rep[key] = dict(avg_us=avg * 1e3, median_us=float(np.median(spans)) * 1e3,
                        min_us=float(np.min(spans)) * 1e3, launches=len(spans),
                        bytes_per_launch=b, gbs=b / (avg * 1e-3) / 1e9,
                        total_ms_per_step=float(np.sum(spans)) / steps)
    return rep


def measure_delayed(args, wl, quant, chunks, inp, torch, D, steps, warmup,
                    stream_stores=True):
    """The pipeline with a one-step delay line for an exchange: two sets of
    per-chunk send buffers alternate by step, and combine of chunk c reads
    the rows packed for chunk c in the previous step (the inputs are the same
    every step, so the result is the same), written some 1.9 GB of traffic
    earlier and long gone from the 256 MB last-level cache: no combine reads
    what the preceding pack just wrote, as on a rank whose rows come back
    from other GPUs.  Same launches as the pipeline (route + layout, pack of
    chunk 0, combine c + pack c+1 merged, combine of the last chunk),
    timed by wall clock over `steps` steps, every write drained inside the
    timed region; then a pass with per-kernel events.  The output is checked
    bit for bit against the ordinary pipeline's.  stream_stores: the send
    rows are written with streaming stores (MOE_PACK_STREAM), the policy for
    rows that are not read back from this GPU's cache.  Step i reads input
    copy i % 2 (Inputs), so its hidden rows and logits are not in that cache
    either."""
    from combine_fp32_router_amd import binding as B

    T, H, E, k, R = wl.T, wl.H, wl.E, wl.k, wl.R
    x_d = inp(0)[0]
    path = D.DispatchCombine(T, H, E, k, R, chunks=chunks, streams=1, ring=1)
    rows = max(path.Tc * k, 1)
    sets = [[B.alloc_rows(rows, H, quant, "cuda") for _ in range(chunks)] for _ in range(2)]
    out = torch.empty_like(x_d)
    caps = path._chunk_caps(wl.capacity_factor) if wl.capacity_factor else None
    rg, vw = path.ranges, path.views
    qp = quant | (B.MOE_PACK_STREAM if stream_stores else 0)

    def step(s, timer=None):
        cur, prev = sets[s % 2], sets[(s + 1) % 2]
        x, lgs = inp(s)
        logits = lgs[0]

        def timed(name, fn):
            tok = timer.start(name, None) if timer else None
            fn()
            if timer:
                timer.stop(tok)

        timed("route_layout", lambda: B.moe_route_layout_chunks(
            logits, k, R, 0, caps, path.idx, path.w, path.lay))
        t0, t1 = rg[0]
        timed("pack", lambda: B.moe_dispatch_pack(x[t0:t1], t1 - t0, H, k, vw[0].pos, qp,
                                                  cur[0][0], cur[0][1]))
        for c in range(chunks - 1):
            (a0, a1), (n0, n1) = rg[c], rg[c + 1]
            timed("combine_pack", lambda: B.moe_combine_pack(
                prev[c][0], prev[c][1], vw[c].pos, path.w[a0:a1], a1 - a0, out[a0:a1],
                x[n0:n1], vw[c + 1].pos, n1 - n0, cur[c + 1][0], cur[c + 1][1], H, k, qp))
        a0, a1 = rg[chunks - 1]
        timed("combine", lambda: B.moe_combine(prev[chunks - 1][0], prev[chunks - 1][1], quant,
                                               vw[chunks - 1].pos, path.w[a0:a1], a1 - a0, H, k,
                                               out[a0:a1]))

    n0 = max(2, warmup)  # the first step fills the delay line; one step counter
    for s in range(n0):  # throughout, so copies and send-buffer sets alternate
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(n0, n0 + steps):
        step(s)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    timer = D.KernelTimer(pool=2 * (3 + chunks) * steps)
    for s in range(n0 + steps, n0 + 2 * steps):
        step(s, timer)
    torch.cuda.synchronize()
    kept = [int(vw[c].expert_offsets[-1].item()) for c in range(chunks)]
    ref = torch.empty_like(x_d)
    path.run(inp(0)[1][0], x_d, ref, quant=quant, capacity_factor=wl.capacity_factor)
    torch.cuda.synchronize()
    same = bool(torch.equal(out, ref))
    byt = step_bytes(wl, [quant], chunks, [kept])
    kr = kernel_report(timer.ms(), wl, [quant], chunks, steps, [kept])
    del path, sets, out, ref
    torch.cuda.empty_cache()
    return {"chunks": chunks, "pack_stores": "streaming" if stream_stores else "device-scope",
            "ms_per_step": round(wall_ms, 4),
            "gbs": round(byt / (wall_ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * byt / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(T / (wall_ms * 1e-3)),
            "algorithmic_bytes_per_step": byt, "output_equals_pipeline": same,
            "kernels": {n: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                            for kk, vv in v.items()} for n, v in kr.items()}}


def measure_swept(wl, quant, chunks, x_d, logits_d, torch, D, flush, steps, warmup):
    """Pack and combine of every chunk as separate launches with the
    last-level cache swept before each (a 1 GiB cached read, untimed), each
    kernel between two HIP events: standalone kernel rates with every input
    byte from HBM.  The sweep after each kernel is timed as well: its excess
    over a sweep of a clean cache ("drain_us") is the kernel's dirty output
    that the cache absorbed during the kernel and wrote back afterwards."""
    from combine_fp32_router_amd import binding as B
    from combine_fp32_router_amd.hipevent import Event

    T, H, E, k, R = wl.T, wl.H, wl.E, wl.k, wl.R
    path = D.DispatchCombine(T, H, E, k, R, chunks=chunks, streams=1, ring=2, merge=False)
    out = torch.empty_like(x_d)
    caps = path._chunk_caps(wl.capacity_factor) if wl.capacity_factor else None

    def rl():
        B.moe_route_layout_chunks(logits_d, k, R, 0, caps, path.idx, path.w, path.lay)

    def pack(c):
        t0, t1 = path.ranges[c]
        st = path.ring[c]
        B.moe_dispatch_pack(x_d[t0:t1], t1 - t0, H, k, st.layout.pos, quant, st.send,
                            st.send_scales)

    def combine(c):
        t0, t1 = path.ranges[c]
        st = path.ring[c]
        B.moe_combine(st.send, st.send_scales, quant, st.layout.pos, path.w[t0:t1], t1 - t0, H,
                      k, out[t0:t1])

    pool = [Event(timing=True) for _ in range(2 * (4 + 4 * chunks) * steps)]
    spans = {}

    def span(name, fn, rec):
        if not rec:
            fn()
            return
        a, b = pool.pop(), pool.pop()
        a.record()
        fn()
        b.record()
        spans.setdefault(name, []).append((a, b))

    for it in range(warmup + steps):
        rec = it >= warmup
        span("flush", flush, rec)
        span("flush_clean", flush, rec)
        span("route_layout", rl, rec)
        span("flush_after_route_layout", flush, rec)
        for c in range(chunks):
            span("pack", lambda: pack(c), rec)
            span("flush_after_pack", flush, rec)
            span("combine", lambda: combine(c), rec)
            span("flush_after_combine", flush, rec)
    torch.cuda.synchronize()
    us = {n: 1e3 * float(np.mean([a.elapsed_ms(b) for a, b in v])) for n, v in spans.items()}
    kept = [int(path.views[c].expert_offsets[-1].item()) for c in range(chunks)]
    ab = algorithmic_bytes(-(-T // chunks), H, E, k, sum(kept) / chunks, quant)
    kern = {}
    for n, b in (("route_layout", algorithmic_bytes(T, H, E, k, T * k, quant)["route_layout"]),
                 ("pack", ab["pack"]), ("combine", ab["combine"])):
        kern[n] = {"avg_us": round(us[n], 2), "bytes_per_launch": int(b),
                   "gbs": round(b / (us[n] * 1e-6) / 1e9, 1),
                   "frac": round(b / (us[n] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "drain_us": round(max(0.0, us[f"flush_after_{n}"] - us["flush_clean"]), 2)}
    del path, out
    torch.cuda.empty_cache()
    return {"chunks": chunks, "sweep_us": round(us["flush_clean"], 2), "kernels": kern}


def snapshot(path, wl, quant, chunks, x_d, logits_d, torch, host_out):
    """GPU results of one more step for the sampled parity check: the whole
    batch's expert ids and weights, and the last chunk's layout, send rows
    (+ scales) and output rows, copied to the host."""
    from combine_fp32_router_amd import binding as B

    out = torch.empty_like(x_d)
    path.run(logits_d, x_d, out, quant=quant)
    torch.cuda.synchronize()
    c = chunks - 1
    t0, t1 = path.ranges[c]
    st = path.chunk_state(c)
    lay = st.layout
    N = int(lay.expert_offsets[-1].item())
    rb = B.moe_row_bytes(wl.H, quant)
    send = st.send.view(-1)[:N * rb].view(N, rb).cpu().numpy()
    scales = st.send_scales[:N].cpu().numpy() if quant else None
    snap = {"quant": quant, "chunks": chunks, "c": c, "t0": t0, "t1": t1,
            "idx": path.idx.cpu().numpy(), "w": path.w.cpu().numpy(),
            "expert_counts": lay.expert_counts.cpu().numpy(),
            "expert_offsets": lay.expert_offsets.cpu().numpy(),
            "rank_counts": lay.rank_counts.cpu().numpy(),
            "rank_offsets": lay.rank_offsets.cpu().numpy(),
            "pos": lay.pos[:(t1 - t0) * wl.k].cpu().numpy(),
            "row_src": lay.row_src[:(t1 - t0) * wl.k].cpu().numpy(),
            "send": send, "scales": scales,
            "out": out[t0:t1].cpu().numpy().view(np.uint16) if host_out else None}
    del out
    return snap


EP_KERNELS = ("recv_layout", "exchange", "regroup", "standin", "ungroup", "exchange_back")


def measure_ep(args, wl, x_d, logits_d, torch):
    """Receiver side with all R ranks on this device (R source shards of T/R
    tokens): per-kernel HIP-event times of the receive layout (offsets and
    row maps), the exchange stand-in, the regroup by expert and its inverse,
    for every payload.  Algorithmic bytes of regroup / ungroup: read + write
    of every kept row and its scale (2*N*S) plus its map entry (4*N); exchange: 2*N*S
    plus the offset tables."""
    from combine_fp32_router_amd import driver as D
    from combine_fp32_router_amd import epgroup as G

    grp = G.EPGroup(wl.T, wl.H, wl.E, wl.k, wl.R, standin=True)
    out = torch.empty_like(x_d)
    res = {"workload": f"{wl.name}: {wl.R} ranks on one device, source shards of "
                       f"{grp.Ts} tokens, stand-in experts on the grouped rows"}
    for quant in ((0, 1, 2, 3) if wl.H % 32 == 0 else (0, 1, 3)):
        for _ in range(args.warmup):
            grp.run(logits_d[0], x_d, out, quant=quant)
        torch.cuda.synchronize()
        N = int(grp.rl.group_offsets[-1].item())
        timer = D.KernelTimer(names=EP_KERNELS, pool=2 * len(EP_KERNELS) * args.steps)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            grp.run(logits_d[0], x_d, out, quant=quant, timer=timer)
        torch.cuda.synchronize()
        layer_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        S = payload_bytes(wl.H, quant)
        tables = 4 * (wl.R * (wl.E + 1) + wl.R * (wl.R + 1) + wl.E * wl.R)
        nbytes = {"recv_layout": tables + 4 * (wl.E + 1) + 8 * N,   # + both row maps
                  "exchange": 2 * N * S + tables, "exchange_back": 2 * N * S + tables,
                  "regroup": 2 * N * S + 4 * N, "ungroup": 2 * N * S + 4 * N,
                  "standin": 2 * N * S + 4 * (wl.E + 1)}
        kr = {}
        for name, spans in timer.ms().items():
            us = 1e3 * sum(spans) / len(spans)
            kr[name] = {"avg_us": round(us, 2), "bytes_per_launch": nbytes[name],
                        "gbs": round(nbytes[name] / (us * 1e-6) / 1e9, 1),
                        "frac_of_8tbs": round(nbytes[name] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        res[PAYLOADS[quant]] = {"rows": N, "payload_bytes_per_row": S,
                                "layer_ms_with_events": round(layer_ms, 4), "kernels": kr}
        log(f"receiver side {PAYLOADS[quant]} N={N} "
            f"{ {k: (v['avg_us'], v['gbs']) for k, v in kr.items()} }")
    del grp
    torch.cuda.empty_cache()
    return res


GEMM_N = 8192  # stand-in expert compute: one bf16 N x N x N GEMM per step


def measure_overlap(args, wl, quants, chunks, inp, torch, D):
    """Dispatch/combine beside a compute kernel (the experts' place, here one
    bf16 GEMM of GEMM_N^3 per step): each alone, both concurrently on two
    ordinary streams, and both concurrently with the data movement confined
    to a quarter, half or three quarters of the CUs and the GEMM to the
    rest (CU-masked streams).  Times are wall clock per step over `steps` steps;
    efficiency = (dc alone + gemm alone) / concurrent."""
    from combine_fp32_router_amd import custreams as CS

    cf = wl.capacity_factor
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=chunks, streams=1, ring=2)
    x_d = inp(0)[0]
    outs = [torch.empty_like(x_d), torch.empty_like(x_d)]
    n = GEMM_N
    a = torch.randn(n, n, dtype=torch.bfloat16, device=x_d.device)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=x_d.device)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=x_d.device)

    count = [0]

    def dc():  # alternating input copies, as in the headline
        x, lgs = inp(count[0])
        count[0] += 1
        run_step(path, lgs, x, outs, quants, cf)

    def gemm():
        torch.matmul(a, b, out=c)

    def timed(pairs):
        """pairs: list of (fn, stream) issued in turn every step."""
        for _ in range(max(1, args.warmup)):
            for fn, st in pairs:
                with torch.cuda.stream(st):
                    fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            for fn, st in pairs:
                with torch.cuda.stream(st):
                    fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    main = torch.cuda.current_stream()
    dc_ms = timed([(dc, main)])
    gemm_ms = timed([(gemm, main)])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    both = {"all_cus": timed([(dc, s1), (gemm, s2)])}
    for q in (1, 2, 3):
        data, comp = CS.split_streams(q)
        try:
            both[f"dc_on_{q}_of_4_cus"] = timed([(dc, data.stream), (gemm, comp.stream)])
        finally:
            data.close()
            comp.close()
    serial = dc_ms + gemm_ms
    res = {"gemm": f"bf16 {n}x{n}x{n} per step on its own stream (stands in for the experts)",
           "dc_alone_ms": round(dc_ms, 4), "gemm_alone_ms": round(gemm_ms, 4),
           "serial_ms": round(serial, 4),
           "concurrent_ms": {k: round(v, 4) for k, v in both.items()},
           "efficiency": {k: round(serial / v, 3) for k, v in both.items()}}
    log(f"overlap dc {dc_ms:.3f} ms + gemm {gemm_ms:.3f} ms = {serial:.3f}; concurrent "
        f"{ {k: round(v, 3) for k, v in both.items()} }")
    del path, a, b, c
    torch.cuda.empty_cache()
    return res


# (workload, payload policy or None for the workload's own, chunks or 0 for
# the workload's own, streams or 0 for the workload's own, steps cap)
CONFIGS = (
    ("mid", (1,), 0, 0, 20),
    ("mid", (0,), 0, 0, 20),
    ("dsv3", (0,), 4, 0, 20),
    ("dsv3", (0,), 1, 0, 20),
    ("dsv3", (1,), 1, 0, 20),
    ("dsv3", (1,), 8, 0, 20),
    ("qwen3", None, 0, 2, 10),
    ("qwen3", None, 0, 1, 10),
    ("large", (0,), 0, 0, 5),
    ("large", (1,), 0, 0, 5),
)


def measure_configs(args, torch, D, I, copy_gbs):
    """The other workloads, wall clock of the whole pipeline (inputs resident
    in HBM), fewer steps than the headline."""
    res = {}
    cache = {}
    for name, quants, chunks, streams, cap in CONFIGS:
        wl = I.WORKLOADS[name]
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            x = I.make_hidden(wl)
            cache[name] = Inputs(torch.from_numpy(x.view(np.int16)).cuda(),
                                 [torch.from_numpy(I.make_logits(wl, l)).cuda()
                                  for l in range(wl.layers)])
            del x
        inp = cache[name]
        x_d = inp(0)[0]
        quants = tuple(quants or wl.quant)
        streams = streams or wl.streams
        chunks = chunks or D.resolve_chunks(wl, quants[0])
        steps, warmup = min(args.steps, cap), min(args.warmup, 3)
        outs = [torch.empty_like(x_d), torch.empty_like(x_d)]
        wall_ms, _, _, kept, path = measure(args, wl, quants, chunks, streams, inp, outs, torch,
                                            D, steps, warmup, kernel_events=False)
        del path, outs
        byt = step_bytes(wl, quants, chunks, kept)
        gbs = byt / (wall_ms * 1e-3) / 1e9
        key = (f"{name}_" + "/".join(PAYLOADS[q] for q in quants) + f"_{chunks}chunks"
               + (f"_{streams}streams" if wl.layers > 1 else ""))
        res[key] = {"T": wl.T, "H": wl.H, "E": wl.E, "k": wl.k, "R": wl.R, "layers": wl.layers,
                    "payload": "/".join(PAYLOADS[q] for q in quants), "chunks": chunks,
                    "streams": streams, "steps": steps, "warmup": warmup,
                    "capacity_factor": (str(wl.capacity_factor) if wl.capacity_factor
                                        else None),
                    "ms_per_step": round(wall_ms, 4), "gbs": round(gbs, 1),
                    "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                    "pct_of_copy_peak": round(100 * gbs / copy_gbs, 2) if copy_gbs else None,
                    "tokens_per_s": round(wl.T / (wall_ms * 1e-3)),
                    "algorithmic_bytes_per_step": byt,
                    "dropped_slots_per_step": sum(wl.T * wl.k - sum(kl) for kl in kept)}
        log(f"config {key}: {wall_ms:.3f} ms/step, {gbs:.1f} GB/s")
    cache.clear()
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ CPU leg
def cpu_threads(requested):
    """Threads for the all-cores leg: the request, else the CPUs this process
    may run on, at most 16 (the host share of one GPU)."""
    if requested > 0:
        return requested
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_leg(wl, quants, chunks, x, logits, threads, snaps, min_seconds=8.0):
    """The oracle as it stands (plain C) on the same work: per step, route the
    batch, then chunk by chunk layout + pack + combine (identity exchange).
    (i) single-threaded, steps repeated until ~min_seconds; (ii) on `threads`
    host threads, the chunk passes of several steps in flight at once (the
    C calls release the interpreter lock).  Throughput on the algorithmic
    bytes of the chunks completed.  Then the sampled parity check: for each
    payload in `snaps`, the oracle's results for the sampled chunk against
    the GPU's."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    bounds = chunk_bounds(wl.T, chunks)
    q = quants[0]

    def chunk_pass(idx, w, t0, t1):
        cap = oracle.capacity_for(t1 - t0, wl.k, wl.E, wl.capacity_factor)
        lay = oracle.dispatch_layout(idx[t0:t1], wl.E, wl.R, cap)
        send = oracle.dispatch_pack(x[t0:t1], lay.pos, q, n_rows=lay.n_rows)
        oracle.combine(send, q, lay.pos, w[t0:t1], wl.H)
        return algorithmic_bytes(t1 - t0, wl.H, wl.E, wl.k, lay.n_rows, q)["total"]

    # (i) single thread
    el, done_bytes, done_chunks, reps = 0.0, 0, 0, 0
    while reps < 8 and el < min_seconds:
        reps += 1
        s = time.perf_counter()
        idx, w = oracle.route_topk(logits[0], wl.k)
        el += time.perf_counter() - s
        for t0, t1 in bounds:
            s = time.perf_counter()
            done_bytes += chunk_pass(idx, w, t0, t1)
            el += time.perf_counter() - s
            done_chunks += 1
            if el >= min_seconds:
                break
    single = dict(value=round(done_bytes / el / 1e9, 4), unit="GB/s", cores=1,
                  seconds=round(el, 3),
                  sample=f"{done_chunks} chunk passes ({len(bounds)} per step, chunks of "
                         f"{bounds[0][1] - bounds[0][0]} tokens, {PAYLOADS[q]} payload): "
                         f"route+layout+pack+combine in {el:.2f} s on one thread")
    per_chunk_s = el / max(done_chunks, 1)
    # (ii) all cores: whole steps, every step's chunk passes in one pool
    steps = max(1, int(round(min_seconds * threads / (per_chunk_s * len(bounds)))))
    steps = min(steps, 64)
    s = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        routes = list(ex.map(lambda _: oracle.route_topk(logits[0], wl.k), range(steps)))
        futs = [ex.submit(chunk_pass, idx, w, t0, t1) for idx, w in routes for t0, t1 in bounds]
        multi_bytes = sum(f.result() for f in futs)
    el_m = time.perf_counter() - s
    base = dict(value=round(multi_bytes / el_m / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle",
                sample=f"{steps} step(s) x {len(bounds)} chunk passes (chunks of "
                       f"{bounds[0][1] - bounds[0][0]} tokens, {PAYLOADS[q]} payload): "
                       f"route+layout+pack+combine in {el_m:.2f} s on {threads} threads "
                       f"(the steps' routes, then all chunk passes, concurrently)"
                       + (" (layer 0 of the stack)" if wl.layers > 1 else ""),
                seconds=round(el_m, 3), host_cpus=os.cpu_count(), cpu_model=cpu_model(),
                single_thread=single)
    log(f"cpu oracle: {single['value']} GB/s on 1 thread, {base['value']} GB/s on "
        f"{threads} threads")
    parity = {name: parity_check(oracle, wl, snap, x, logits[0])
              for name, snap in snaps.items()}
    return base, parity


def _codes(rows, H, quant):
    """Signed integer image of a row buffer's codes: int8 as is, int4 nibbles
    (element 2i in the low nibble), E4M3 as sign-magnitude (neighbouring codes
    differ by one)."""
    if quant == 1:
        return rows[:, :H].view(np.int8).astype(np.int32)
    if quant == 2:
        b = rows[:, :H // 2].astype(np.int32)
        c = np.empty((rows.shape[0], H), dtype=np.int32)
        c[:, 0::2], c[:, 1::2] = b & 0xF, b >> 4
        return np.where(c >= 8, c - 16, c)
    b = rows[:, :H].astype(np.int32)
    return np.where(b & 0x80, -(b & 0x7F), b & 0x7F)


def parity_check(oracle, wl, snap, x, logits):
    """The GPU's results of one step against the oracle: expert ids and
    weights for the whole batch; layout, send rows (+ scales) and combined
    output rows of the sampled chunk (the oracle's combine reads the
    oracle's own send rows).  Bars: ids, layouts and bf16 rows bit-exact;
    codes within +-1 (mismatch count reported); weights 1e-6 relative;
    outputs 1e-3 + 1e-2*|ref| element-wise."""
    H, k, q = wl.H, wl.k, snap["quant"]
    t0, t1 = snap["t0"], snap["t1"]
    idx_ref, w_ref = oracle.route_topk(logits, k)
    res = {"chunk": snap["c"], "tokens": [t0, t1],
           "ids_mismatches": int((snap["idx"][:wl.T] != idx_ref).sum()),
           "weights_max_rel_err": weights_max_rel_err(snap["w"][:wl.T], w_ref)}
    cap = oracle.capacity_for(t1 - t0, k, wl.E, wl.capacity_factor)
    lay = oracle.dispatch_layout(idx_ref[t0:t1], wl.E, wl.R, cap)
    N = lay.n_rows
    lm = 0
    for name, ref in (("expert_counts", lay.expert_counts), ("expert_offsets", lay.expert_offsets),
                      ("rank_counts", lay.rank_counts), ("rank_offsets", lay.rank_offsets),
                      ("pos", lay.pos.ravel()), ("row_src", lay.row_src)):
        lm += int((snap[name].ravel()[:ref.size] != ref.ravel()).sum())
    res["layout_mismatches"] = lm
    send_ref = oracle.dispatch_pack(x[t0:t1], lay.pos, q, n_rows=N)
    rb = snap["send"].shape[1]
    g = snap["send"][:N]
    if q == 0:
        res["rows"] = N
        res["bf16_element_mismatches"] = int((g.view(np.uint16) != send_ref[:, :rb]
                                              .view(np.uint16)).sum())
    else:
        d = np.abs(_codes(g, H, q) - _codes(send_ref, H, q))
        sg = snap["scales"][:N].view(np.int32).astype(np.int64)
        sr = send_ref[:, rb:rb + 4].copy().view(np.int32).ravel().astype(np.int64)
        res.update(rows=N, codes=int(d.size), code_mismatches=int((d != 0).sum()),
                   max_code_diff=int(d.max(initial=0)),
                   scale_max_ulp_diff=int(np.abs(sg - sr).max(initial=0)))
    out_ref = oracle.combine(send_ref, q, lay.pos, w_ref[t0:t1], H)
    with np.errstate(invalid="ignore"):
        gf = (snap["out"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rf = (out_ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        err = np.abs(gf - rf)
        fin = np.isfinite(err)
        big = fin & (np.abs(rf) > 1e-2)
        res.update(out_elements=int(err.size), out_nonfinite=int((~fin).sum()),
                   out_max_abs_err=float(err[fin].max(initial=0.0)),
                   out_max_rel_err=float((err[big] / np.abs(rf[big])).max(initial=0.0)),
                   out_rel_err_over="elements with |ref| > 1e-2",
                   # a NaN fails the bar too
                   out_violations=int((~(err <= 1e-3 + 1e-2 * np.abs(rf))).sum()))
    ok = (res["ids_mismatches"] == 0 and res["layout_mismatches"] == 0
          and res["weights_max_rel_err"] <= 1e-6 and res["out_violations"] == 0
          and (res.get("bf16_element_mismatches", 0) == 0)
          and res.get("max_code_diff", 0) <= 1 and res.get("scale_max_ulp_diff", 0) <= 1)
    res["pass"] = bool(ok)
    log(f"parity {PAYLOADS[q]} chunk {snap['c']}: {res}")
    return res


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no cross-GPU step "
              "(multi-GPU sharding is described, not implemented); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from combine_fp32_router_amd import binding as B
    from combine_fp32_router_amd import driver as D
    from combine_fp32_router_amd import harness as HN
    from combine_fp32_router_amd import inputs as I

    B.load()
    HN.load()
    if args.copy_probe > 0:
        print(json.dumps(probe_peaks(torch, int(args.copy_probe * (1 << 30)) // 16 * 16)),
              flush=True)
        return
    wl = I.WORKLOADS[args.workload]
    streams = args.streams or wl.streams
    log(f"{wl.name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} layers={wl.layers} "
        f"chunks={args.chunks or wl.chunks or 'fitted'} streams={streams} "
        f"steps={args.steps} warmup={args.warmup}")
    peaks = probe_peaks(torch)
    copy_gbs = peaks["copy_gbs"]
    x = I.make_hidden(wl)
    logits = [I.make_logits(wl, l) for l in range(wl.layers)]
    dev = torch.device("cuda:0")
    x_d = torch.from_numpy(x.view(np.int16)).to(dev)
    logits_d = [torch.from_numpy(lg).to(dev) for lg in logits]
    inp = Inputs(x_d, logits_d)
    outs = [torch.empty_like(x_d), torch.empty_like(x_d)]
    torch.cuda.synchronize()

    if wl.layers > 1:  # the workload's own per-layer payload policy
        policies = {"policy": list(wl.quant)}
        primary = "policy"
    else:
        q0 = args.quant if args.quant is not None else wl.quant[0]
        policies = {PAYLOADS[q0]: [q0]}
        if not args.no_variant:
            for q in (0, 1, 2, 3):
                if q != q0 and (q != 2 or wl.H % 32 == 0):
                    policies[PAYLOADS[q]] = [q]
        primary = PAYLOADS[q0]
    results, snaps = {}, {}
    flush = None if args.no_cold else Flush(torch)
    for name, quants in policies.items():
        chunks = args.chunks or D.resolve_chunks(wl, quants[0])
        wall_ms, gpu_ms, kms, kept, path = measure(
            args, wl, quants, chunks, streams, inp, outs, torch, D, args.steps,
            args.warmup, kernel_events=not args.no_kernel_events)
        if wl.layers == 1 and not args.no_cpu_baseline:
            snaps[name] = snapshot(path, wl, quants[0], chunks, x_d, logits_d[0], torch, True)
        del path
        byt = step_bytes(wl, quants, chunks, kept)
        kr = kernel_report(kms, wl, quants, chunks, args.steps, kept)
        dropped = sum(wl.T * wl.k - sum(kl) for kl in kept)
        results[name] = dict(wall_ms=wall_ms, gpu_ms=gpu_ms, bytes=byt, kernels=kr, quants=quants,
                             chunks=chunks,
                             gbs=byt / (wall_ms * 1e-3) / 1e9, dropped=dropped,
                             tokens_per_s=wl.T / (wall_ms * 1e-3))
        log(f"{name} chunks={chunks} {wall_ms:.3f} ms/step, {results[name]['gbs']:.1f} GB/s "
            f"kernels={ {k: round(v['avg_us'], 1) for k, v in kr.items()} }")
        if flush is not None and wl.layers == 1:
            cold = measure_delayed(args, wl, quants[0], chunks, inp, torch, D,
                                   args.steps, args.warmup, stream_stores=True)
            dev_st = measure_delayed(args, wl, quants[0], chunks, inp, torch, D,
                                     args.steps, args.warmup, stream_stores=False)
            cold["device_scope_pack_stores"] = {k: dev_st[k] for k in
                                                ("ms_per_step", "gbs", "pct_of_peak",
                                                 "output_equals_pipeline")}
            cold["kernels_swept"] = measure_swept(wl, quants[0], chunks, x_d, logits_d[0], torch,
                                                  D, flush, min(args.steps, 20),
                                                  min(args.warmup, 3))
            results[name]["cold"] = cold
            sw = cold["kernels_swept"]["kernels"]
            log(f"{name} cache-cold (delay line, streaming stores): {cold['ms_per_step']:.3f} "
                f"ms/step, {cold['gbs']} GB/s ({cold['pct_of_peak']}%), same output "
                f"{cold['output_equals_pipeline']}; device-scope stores "
                f"{dev_st['ms_per_step']:.3f} ms/step; kernels "
                f"{ {k: round(v['avg_us'], 1) for k, v in cold['kernels'].items()} }; swept "
                f"{ {k: (v['avg_us'], v['drain_us']) for k, v in sw.items()} }")
        torch.cuda.empty_cache()

    r = results[primary]
    chunks = r["chunks"]
    roof = None
    if r["kernels"]:
        big = {k: v for k, v in r["kernels"].items()
               if k.split("@")[0] in ("pack", "combine", "combine_pack")}
        dom = max(big, key=lambda n: big[n]["total_ms_per_step"])
        kd = big[dom]
        kname = dom.split("@")[0]
        layer = int(dom.split("@")[1][1:]) if "@" in dom else 0
        tr = load_traffic(kname, wl.name, r["quants"][layer])
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(kd["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kd["gbs"] / HBM_PEAK_GBS, 4),
                "traffic": None if tr is None else tr.get("bytes_per_launch"),
                "avg_launch_us": round(kd["avg_us"], 2),
                "median_launch_us": round(kd["median_us"], 2),
                "min_launch_us": round(kd["min_us"], 2),
                "algorithmic_bytes_per_launch": kd["bytes_per_launch"],
                "frac_of_copy_peak": round(kd["gbs"] / copy_gbs, 4)}
        if "cold" in r:
            ck = {n: v for n, v in r["cold"]["kernels"].items()
                  if n in ("pack", "combine", "combine_pack")}
            cdom = max(ck, key=lambda n: ck[n]["total_ms_per_step"])
            roof["hbm_cold"] = {
                "kernel": cdom, "achieved": round(ck[cdom]["gbs"], 1),
                "frac": round(ck[cdom]["gbs"] / HBM_PEAK_GBS, 4),
                "avg_launch_us": round(ck[cdom]["avg_us"], 2),
                "median_launch_us": round(ck[cdom]["median_us"], 2),
                "min_launch_us": round(ck[cdom]["min_us"], 2),
                "algorithmic_bytes_per_launch": ck[cdom]["bytes_per_launch"],
                "frac_of_copy_peak": round(ck[cdom]["gbs"] / copy_gbs, 4),
                "note": "the dominant kernel of the delay-line pipeline (hbm_cold): its combine "
                        "half reads rows written a step earlier, from HBM"}
    payload = "/".join(PAYLOADS[q] for q in r["quants"])
    desc = (f"{wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R}, "
            + (f"{wl.layers} layers, " if wl.layers > 1 else "")
            + f"{chunks} chunks"
            + ("" if (args.chunks or wl.chunks) else " (fitted to the 256 MB last-level cache)")
            + f", {payload} payload, {streams} stream(s)"
            + ("" if args.no_merge or streams == 3 or args.ring < 2
               else ", combine of chunk c and pack of chunk c+1 in one launch")
            + (", Zipf(1.1) expert bias, 1% rows x50" if wl.zipf_s else "")
            + (f", capacity factor {wl.capacity_factor}" if wl.capacity_factor else ""))
    line = {
        "metric": METRIC,
        "value": round(r["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": payload if wl.layers > 1 else PAYLOADS[r["quants"][0]],
        "data": "synthetic",
        "config": {"workload": desc, "T": wl.T, "H": wl.H, "E": wl.E, "k": wl.k, "R": wl.R,
                   "layers": wl.layers, "chunks": chunks, "payload": payload,
                   "streams": streams, "merged": not (args.no_merge or streams == 3
                                                       or args.ring < 2),
                   "hip_graph": bool(args.graph)},
        "pct_of_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2),
        "pct_of_copy_peak": round(100 * r["gbs"] / copy_gbs, 2),
        "tokens_per_s": round(r["tokens_per_s"]),
        "gpu_event_ms_per_step": round(r["gpu_ms"], 4),
        "algorithmic_bytes_per_step": r["bytes"],
        "dropped_slots_per_step": r["dropped"],
        "roofline": roof,
        "copy_peak": peaks,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in r["kernels"].items()},
        "variants": {},
    }
    if "cold" in r:
        cold = dict(r["cold"])
        cold["pct_of_copy_peak"] = round(100 * cold["gbs"] / copy_gbs, 2)
        cold["note"] = ("HBM-only figure: the same pipeline and launches, but combine of chunk "
                        "c reads the rows packed for chunk c one step earlier (two alternating "
                        "sets of send buffers), so none of its reads can come from the "
                        "last-level cache; the pack writes its rows with streaming stores "
                        "(MOE_PACK_STREAM, the policy for rows not read back from this GPU's "
                        "cache; device_scope_pack_stores: the same with the default policy); "
                        "wall clock per step, all writes drained inside the timed region.  value "
                        "and roofline.frac are the ordinary pipeline, whose combines read much of "
                        "their rows from that cache.  kernels_swept: pack and combine launched "
                        "alone after a cache sweep")
        line["hbm_cold"] = cold
    for name, rr in results.items():
        if name == primary:
            continue
        v = {"value": round(rr["gbs"], 1), "unit": "GB/s", "ms_per_step": round(rr["wall_ms"], 4),
             "chunks": rr["chunks"],
             "pct_of_peak": round(100 * rr["gbs"] / HBM_PEAK_GBS, 2),
             "pct_of_copy_peak": round(100 * rr["gbs"] / copy_gbs, 2),
             "tokens_per_s": round(rr["tokens_per_s"]),
             "algorithmic_bytes_per_step": rr["bytes"],
             "payload_bytes_ratio_vs_bf16": round(payload_bytes(wl.H, rr["quants"][0]) / (2 * wl.H),
                                                  4),
             "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                             for kk, vv in v.items()} for k, v in rr["kernels"].items()}}
        if "cold" in rr:
            v["hbm_cold"] = rr["cold"]
        line["variants"][name] = v
    if not args.no_configs and args.workload == "dsv3":
        line["configs"] = measure_configs(args, torch, D, I, copy_gbs)
    if not args.no_ep and wl.layers == 1:
        line["receiver_side"] = measure_ep(args, wl, x_d, logits_d, torch)
    if not args.no_overlap:
        line["overlap"] = measure_overlap(args, wl, r["quants"], chunks, inp, torch, D)
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline_leg(wl, r["quants"], chunks, x, logits,
                                        cpu_threads(args.cpu_threads), snaps)
        base["gpu_over_oracle"] = round(r["gbs"] / base["value"], 1)
        line["cpu_baseline"] = base
        if parity:
            line["parity"] = parity
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
