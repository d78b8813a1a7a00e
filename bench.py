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
(GB/s, 1e9 bytes).  Algorithmic bytes per layer (N = kept rows, S = bytes
a row carries: 2H for bf16, H codes + a 4-byte scale for int8 and fp8, H/2
+ 4 for int4):
  route    T*E*4 + T*k*8
  layout   T*k*4 + 2*T*k*4
  pack     T*H*2 + T*k*4 + N*S
  combine  N*S + T*k*8 + T*H*2
The 2*N*S part is the 2*T*k*H*b exchange volume of the communication-wall
explainer.

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
    ap.add_argument("--no-variant", action="store_true", help="skip the other payload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the dispatch/combine + concurrent GEMM measurement")
    ap.add_argument("--no-ep", action="store_true",
                    help="skip the receiver-side (all ranks on one device) measurement")
    ap.add_argument("--json-out", default="")
    ap.add_argument("--copy-probe", type=float, default=0.0,
                    help="only run the plain copy kernel over this many GiB (achievable "
                         "bandwidth and counter calibration) and exit")
    return ap.parse_args()


def copy_probe(args):
    """Plain 16-byte copy of a known size: read + write bytes / kernel time."""
    import torch

    from combine_fp32_router_amd import binding as B

    nbytes = int(args.copy_probe * (1 << 30)) // 16 * 16
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        B.moe_copy_probe(src, dst, nbytes)
    from combine_fp32_router_amd.hipevent import Event

    evs = [(Event(timing=True), Event(timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        B.moe_copy_probe(src, dst, nbytes)
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_ms(b) for a, b in evs]
    assert torch.equal(src[:4096], dst[:4096]) and torch.equal(src[-4096:], dst[-4096:])
    line = {"probe": "copy", "bytes_per_launch": 2 * nbytes, "launches": len(ms),
            "avg_us": round(1e3 * float(np.mean(ms)), 2), "min_us": round(1e3 * min(ms), 2),
            "gbs_avg": round(2 * nbytes / (np.mean(ms) * 1e-3) / 1e9, 1),
            "gbs_best": round(2 * nbytes / (min(ms) * 1e-3) / 1e9, 1)}
    print(json.dumps(line), flush=True)


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


def measure(args, wl, quants, chunks, streams, x_d, logits_list, outs, torch, D):
    """Warm up, then time exactly `steps` steps with nothing else on the
    stream (wall clock + one event pair around the whole region).  Then run
    the same number of steps again with HIP events around every launch, on
    the launch's own stream, for the per-kernel durations: a recorded event
    delays the next kernel by several microseconds, so per-kernel events stay
    out of the wall-clock region.  Returns the kept rows of every layer's
    chunks (read after the timed region)."""
    from combine_fp32_router_amd.hipevent import Event

    cf = wl.capacity_factor
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=chunks, streams=streams,
                             ring=args.ring, fused=not args.unfused, merge=not args.no_merge)
    step = lambda: run_step(path, logits_list, x_d, outs, quants, cf)  # noqa: E731
    if args.graph:
        if streams == 3:
            raise SystemExit("--graph captures the one- and two-stream paths")
        graph = D.capture(step)
        step = graph.replay
    for _ in range(args.warmup):
        step()
    ev0, ev1 = Event(timing=True), Event(timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    gpu_ms = ev0.elapsed_ms(ev1) / args.steps
    kms = {}
    if not args.no_kernel_events:
        launches = len(quants) * (2 + 3 * chunks)
        timer = D.KernelTimer(pool=2 * launches * args.steps)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            run_step(path, logits_list, x_d, outs, quants, cf, timer=timer)
        torch.cuda.synchronize()
        kms = timer.ms()
    # kept rows per layer and chunk (capacity may drop some): one more step,
    # layer by layer, reading each layer's expert offsets
    kept = []
    cur = x_d
    for l, (lg, q) in enumerate(zip(logits_list, quants)):
        path.run(lg, cur, outs[l % 2], quant=q, capacity_factor=cf)
        cur = outs[l % 2]
        torch.cuda.synchronize()
        kept.append([int(path.views[c].expert_offsets[-1].item()) for c in range(chunks)])
    return wall_ms, gpu_ms, kms, kept


def step_bytes(wl, quants, chunks, kept):
    """Algorithmic bytes of one step, summed over layers and chunks."""
    tot = 0
    for q, kl in zip(quants, kept):
        for c, (t0, t1) in enumerate(chunk_bounds(wl.T, chunks)):
            b = algorithmic_bytes(t1 - t0, wl.H, wl.E, wl.k, kl[c], q)
            tot += b["total"]
    return tot


def chunk_bounds(T, chunks):
    step = -(-T // chunks)
    return [(min(T, c * step), min(T, (c + 1) * step)) for c in range(chunks)]


def kernel_report(kms, wl, quants, chunks, steps, kept):
    """Average launch duration and achieved GB/s per kernel: algorithmic
    bytes of one launch / its HIP-event duration.  Keys are the kernel name,
    or name@L<layer> for multi-layer steps."""
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
        rep[key] = dict(avg_us=avg * 1e3, launches=len(spans), bytes_per_launch=b,
                        gbs=b / (avg * 1e-3) / 1e9,
                        total_ms_per_step=float(np.sum(spans)) / steps)
    return rep


EP_KERNELS = ("recv_layout", "exchange", "regroup", "standin", "ungroup", "exchange_back")


def measure_ep(args, wl, x_d, logits_d, torch):
    """Receiver side with all R ranks on this device (R source shards of T/R
    tokens): per-kernel HIP-event times of the receive layout (offsets and
    row maps), the exchange stand-in, the regroup by expert and its inverse,
    for both payloads.  Algorithmic bytes of regroup / ungroup: read + write
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
                                                 "layer_ms_with_events": round(layer_ms, 4),
                                                 "kernels": kr}
        print(f"bench: receiver side {PAYLOADS[quant]} N={N} "
              f"{ {k: (v['avg_us'], v['gbs']) for k, v in kr.items()} }",
              file=sys.stderr, flush=True)
    del grp
    torch.cuda.empty_cache()
    return res


GEMM_N = 8192  # stand-in expert compute: one bf16 N x N x N GEMM per step


def measure_overlap(args, wl, quants, chunks, x_d, logits_d, torch, D):
    """Dispatch/combine beside a compute kernel (the experts' place, here one
    bf16 GEMM of GEMM_N^3 per step): each alone, both concurrently on two
    ordinary streams, and both concurrently with the data movement confined
    to a quarter, half or three quarters of the CUs and the GEMM to the
    rest (CU-masked streams).  Times are wall clock per step over `steps` steps;
    efficiency = (dc alone + gemm alone) / concurrent."""
    from combine_fp32_router_amd import custreams as CS

    cf = wl.capacity_factor
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=chunks, streams=1, ring=2)
    outs = [torch.empty_like(x_d), torch.empty_like(x_d)]
    n = GEMM_N
    a = torch.randn(n, n, dtype=torch.bfloat16, device=x_d.device)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=x_d.device)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=x_d.device)

    def dc():
        run_step(path, logits_d, x_d, outs, quants, cf)

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
    print(f"bench: overlap dc {dc_ms:.3f} ms + gemm {gemm_ms:.3f} ms = {serial:.3f}; concurrent "
          f"{ {k: round(v, 3) for k, v in both.items()} }", file=sys.stderr, flush=True)
    del path, a, b, c
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, quants, chunks, x, logits_list, min_seconds=10.0, max_reps=8):
    """The oracle as it stands (plain single-threaded C) on the same work:
    per layer, route the batch, then chunk by chunk layout + pack + combine
    (identity exchange), layer l+1 on the oracle's own layer-l output.  The
    step is repeated until ~min_seconds of CPU time (at most max_reps
    times), stopping early after the chunk that passes min_seconds; the
    throughput is on the algorithmic bytes of the chunks completed."""
    import oracle

    el, done_bytes, done_chunks, reps = 0.0, 0, 0, 0
    bounds = chunk_bounds(wl.T, chunks)
    while reps < max_reps and el < min_seconds:
        reps += 1
        cur = x
        for q, lg in zip(quants, logits_list):
            out = np.zeros_like(cur)
            s = time.perf_counter()
            idx, w = oracle.route_topk(lg, wl.k)
            el += time.perf_counter() - s
            for t0, t1 in bounds:
                s = time.perf_counter()
                cap = oracle.capacity_for(t1 - t0, wl.k, wl.E, wl.capacity_factor)
                lay = oracle.dispatch_layout(idx[t0:t1], wl.E, wl.R, cap)
                send = oracle.dispatch_pack(cur[t0:t1], lay.pos, q, n_rows=lay.n_rows)
                out[t0:t1] = oracle.combine(send, q, lay.pos, w[t0:t1], wl.H)
                el += time.perf_counter() - s
                done_bytes += algorithmic_bytes(t1 - t0, wl.H, wl.E, wl.k, lay.n_rows, q)["total"]
                done_chunks += 1
                if el >= min_seconds:
                    break
            if el >= min_seconds:
                break
            cur = out
    return dict(value=round(done_bytes / el / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"{done_chunks} chunk passes over {reps} repetition(s) of the step "
                       f"({len(quants) * chunks} passes per step: chunks of "
                       f"{bounds[0][1] - bounds[0][0]} tokens, payload per layer "
                       f"{list(quants)}): route+layout+pack+combine in {el:.2f} s of "
                       f"single-threaded C",
                seconds=round(el, 3), host_cpus=os.cpu_count())


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no cross-GPU step "
              "(multi-GPU sharding is described, not implemented); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe > 0:
        copy_probe(args)
        return
    import torch

    from combine_fp32_router_amd import binding as B
    from combine_fp32_router_amd import driver as D
    from combine_fp32_router_amd import inputs as I

    B.load()
    wl = I.WORKLOADS[args.workload]
    streams = args.streams or wl.streams
    print(f"bench: {wl.name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} layers={wl.layers} "
          f"chunks={args.chunks or wl.chunks or 'fitted'} streams={streams} "
          f"steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    x = I.make_hidden(wl)
    logits = [I.make_logits(wl, l) for l in range(wl.layers)]
    dev = torch.device("cuda:0")
    x_d = torch.from_numpy(x.view(np.int16)).to(dev)
    logits_d = [torch.from_numpy(lg).to(dev) for lg in logits]
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
    results = {}
    for name, quants in policies.items():
        chunks = args.chunks or D.resolve_chunks(wl, quants[0])
        wall_ms, gpu_ms, kms, kept = measure(args, wl, quants, chunks, streams, x_d, logits_d,
                                             outs, torch, D)
        byt = step_bytes(wl, quants, chunks, kept)
        kr = kernel_report(kms, wl, quants, chunks, args.steps, kept)
        dropped = sum(wl.T * wl.k - sum(kl) for kl in kept)
        results[name] = dict(wall_ms=wall_ms, gpu_ms=gpu_ms, bytes=byt, kernels=kr, quants=quants,
                             chunks=chunks,
                             gbs=byt / (wall_ms * 1e-3) / 1e9, dropped=dropped,
                             tokens_per_s=wl.T / (wall_ms * 1e-3))
        print(f"bench: {name} chunks={chunks} {wall_ms:.3f} ms/step, "
              f"{results[name]['gbs']:.1f} GB/s "
              f"kernels={ {k: round(v['avg_us'], 1) for k, v in kr.items()} }",
              file=sys.stderr, flush=True)
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
                "algorithmic_bytes_per_launch": kd["bytes_per_launch"]}
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
        "tokens_per_s": round(r["tokens_per_s"]),
        "gpu_event_ms_per_step": round(r["gpu_ms"], 4),
        "algorithmic_bytes_per_step": r["bytes"],
        "dropped_slots_per_step": r["dropped"],
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in r["kernels"].items()},
        "variants": {},
    }
    for name, rr in results.items():
        if name == primary:
            continue
        line["variants"][name] = {
            "value": round(rr["gbs"], 1), "unit": "GB/s", "ms_per_step": round(rr["wall_ms"], 4),
            "chunks": rr["chunks"],
            "pct_of_peak": round(100 * rr["gbs"] / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(rr["tokens_per_s"]),
            "algorithmic_bytes_per_step": rr["bytes"],
            "payload_bytes_ratio_vs_bf16": round(payload_bytes(wl.H, rr["quants"][0]) / (2 * wl.H),
                                                 4),
            "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                            for kk, vv in v.items()} for k, v in rr["kernels"].items()}}
    if not args.no_ep and wl.layers == 1:
        line["receiver_side"] = measure_ep(args, wl, x_d, logits_d, torch)
    if not args.no_overlap:
        line["overlap"] = measure_overlap(args, wl, r["quants"], chunks, x_d, logits_d, torch, D)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, r["quants"], chunks, x, logits)
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
