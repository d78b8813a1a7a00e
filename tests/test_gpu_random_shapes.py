"""Seeded random-shape parity sweep: whole layers through the default
driver (route+layout fused, merged combine+pack launches, one stream) on
shapes drawn within the documented limits -- T, H, E, k, R, chunk count,
payload, capacity factor, Zipf-skewed routing and outlier rows -- against
the oracle's chunked layer: expert ids bit-exact, per-chunk counts and
offsets bit-exact, gate weights within 1e-6 relative, outputs within
1e-3 + 1e-2 |ref|.  Shapes are small enough for the oracle to finish in
seconds; the draws are fixed by the seed, so a failure names a
reproducible case."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I
from gpu_util import (assert_out_close, assert_weights, compare_records, dev, host,
                      host_records)

pytestmark = pytest.mark.gpu


def draw_cases(n=40, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        R = int(rng.choice([1, 2, 4, 8, 16]))
        E = R * int(rng.integers(1, 1024 // R + 1))            # E % R == 0, E <= 1024
        k = int(rng.integers(1, min(E, 16) + 1))
        quant = int(rng.integers(0, 4))
        H = 32 * int(rng.integers(1, 96))                      # H % 32 == 0: every payload
        T = int(rng.integers(1, 3000))
        T = max(1, min(T, 20_000_000 // (k * H)))              # oracle work stays seconds
        chunks = int(rng.integers(1, 9))
        cf = [None, Fraction(1), Fraction(5, 4)][int(rng.integers(0, 3))]
        zipf = [None, 1.1][int(rng.integers(0, 2))]
        outl = [0.0, 0.01][int(rng.integers(0, 2))]
        cases.append((f"r{i}", T, H, E, k, R, chunks, quant, cf, zipf, outl))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("name,T,H,E,k,R,chunks,quant,cf,zipf,outl", CASES,
                         ids=[f"{c[0]}-T{c[1]}-H{c[2]}-E{c[3]}-k{c[4]}-C{c[6]}-q{c[7]}" for c in CASES])
def test_random_layer(name, T, H, E, k, R, chunks, quant, cf, zipf, outl):
    wl = I.Workload(name, T=T, H=H, E=E, k=k, R=R, zipf_s=zipf, outlier_frac=outl, seed=17)
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    ref = oracle.run_layer(logits, x, E, k, R, chunks=chunks, quant=quant, capacity_factor=cf,
                           keep_buffers=False)
    path = D.DispatchCombine(T, H, E, k, R, chunks=chunks)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    path.run(dev(logits), dev(x), out, quant=quant, capacity_factor=cf)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(path.idx)[:T], ref.idx)
    assert_weights(host(path.w)[:T], ref.w)
    # chunks past the last token (chunks > T) have no layout on the device
    nonempty = [c for c, (t0, t1) in enumerate(D.chunk_ranges(T, chunks)) if t1 > t0]
    for c in nonempty:
        lay = ref.layouts[c]
        np.testing.assert_array_equal(host(path.views[c].expert_counts), lay.expert_counts)
        np.testing.assert_array_equal(host(path.views[c].expert_offsets), lay.expert_offsets)
    assert_out_close(host(out), ref.out, f"{name} q{quant} C{chunks} cf={cf}")


@pytest.mark.parametrize("name,T,H,E,k,R,chunks,quant,cf,zipf,outl", CASES[:12],
                         ids=[f"{c[0]}-T{c[1]}-H{c[2]}-E{c[3]}-k{c[4]}-C{c[6]}-q{c[7]}" for c in CASES[:12]])
def test_random_layer_two_streams_standin(name, T, H, E, k, R, chunks, quant, cf, zipf, outl):
    """The same draws on the two-stream driver with the stand-in expert
    between dispatch and combine (re-quantised on the return path)."""
    wl = I.Workload(name, T=T, H=H, E=E, k=k, R=R, zipf_s=zipf, outlier_frac=outl, seed=18)
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    ref = oracle.run_layer(logits, x, E, k, R, chunks=chunks, quant=quant, capacity_factor=cf,
                           standin=True, keep_buffers=False)
    path = D.DispatchCombine(T, H, E, k, R, chunks=chunks, streams=2, standin=True)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    path.run(dev(logits), dev(x), out, quant=quant, capacity_factor=cf)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(path.idx)[:T], ref.idx)
    assert_out_close(host(out), ref.out, f"{name} two streams, stand-in, q{quant}")


@pytest.mark.parametrize("name,T,H,E,k,R,chunks,quant,cf,zipf,outl", CASES[12:24],
                         ids=[f"{c[0]}-T{c[1]}-H{c[2]}-E{c[3]}-k{c[4]}-R{c[5]}-q{c[7]}" for c in CASES[12:24]])
def test_random_ep_group(name, T, H, E, k, R, chunks, quant, cf, zipf, outl):
    """The same kind of draws through the receiver side: R source shards on
    one device, exchange stand-in, regroup by expert, stand-in experts,
    ungroup, return exchange, per-source combine -- against the oracle's
    R-rank layer (offsets, grouped offsets and bf16 grouped rows bit-exact,
    quantised grouped rows to the pack's bar, outputs within the bar)."""
    from combine_fp32_router_amd import epgroup as G

    wl = I.Workload(name, T=T, H=H, E=E, k=k, R=R, zipf_s=zipf, outlier_frac=outl, seed=19)
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    ref = oracle.run_ep_layer(logits, x, E, k, R, quant=quant, capacity_factor=cf)
    grp = G.EPGroup(T, H, E, k, R, standin=True)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    grp.run(dev(logits), dev(x), out, quant=quant, capacity_factor=cf)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(grp.rl.group_offsets), ref.rl.group_offsets)
    np.testing.assert_array_equal(host(grp.src_offsets),
                                  np.stack([lay.expert_offsets for lay in ref.layouts]))
    N = ref.rl.n_rows
    got = host_records(grp.grouped, grp.grouped_scales, N, H, quant)
    if quant == 0:
        np.testing.assert_array_equal(got, ref.grouped[:N])
    else:
        compare_records(got, ref.grouped[:N], H, quant, f"{name} grouped")
    assert_out_close(host(out), ref.out, f"{name} R={R} q{quant}")
