"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: expert ids, counts, offsets, pos and row_src bit-exact; bf16 rows
bit-exact; int8 codes within +-1 (mismatch count reported, 0 expected) and
scales within 1 ulp; gate weights within 1e-6 relative; combined bf16 output
within 1e-3 absolute + 1e-2 relative of the oracle, element by element.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_fp32_router_amd import binding as B
from combine_fp32_router_amd import harness as HN
from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I

from gpu_util import (assert_out_close, assert_weights, compare_records, dev, host,
                      host_records, join_records, row_bytes, sampled_records)

pytestmark = pytest.mark.gpu

# ------------------------------------------------------------------ route
ROUTE_CASES = [
    ("tiny", None), ("mid", None), ("dsv3", None),
    ("T1", I.Workload("T1", T=1, H=16, E=8, k=2, R=2)),
    ("ragged", I.Workload("ragged", T=1001, H=16, E=37, k=5, R=1)),
    ("E1024", I.Workload("E1024", T=333, H=16, E=1024, k=16, R=8)),
    ("k1", I.Workload("k1", T=500, H=16, E=64, k=1, R=8)),
    ("kE", I.Workload("kE", T=300, H=16, E=8, k=8, R=4)),
    ("E200", I.Workload("E200", T=700, H=16, E=200, k=6, R=5)),
    ("E300", I.Workload("E300", T=257, H=16, E=300, k=7, R=3)),
    ("E301", I.Workload("E301", T=257, H=16, E=301, k=7, R=7)),
    ("E36", I.Workload("E36", T=999, H=16, E=36, k=3, R=4)),
    # 32-bit fast selection (E = 128 / 256, k <= 8) with a ragged last block
    ("E256_ragged", I.Workload("E256_ragged", T=1001, H=16, E=256, k=8, R=8)),
    ("E128_k6_ragged", I.Workload("E128_k6_ragged", T=77, H=16, E=128, k=6, R=4)),
    ("E256_k1", I.Workload("E256_k1", T=301, H=16, E=256, k=1, R=8)),
]


@pytest.mark.parametrize("name,wl", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_parity(name, wl):
    wl = wl or I.WORKLOADS[name]
    logits = I.make_logits(wl)
    idx_ref, w_ref = oracle.route_topk(logits, wl.k)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    B.moe_route_topk(dev(logits), wl.k, idx, w)
    np.testing.assert_array_equal(host(idx), idx_ref)
    assert_weights(host(w), w_ref)


@pytest.mark.parametrize("E", [64, 200, 256, 512])
def test_route_unaligned_rows(E):
    """Logits starting 4 bytes past a 16-byte boundary take the 4-byte-load
    path; results must not depend on which path ran."""
    wl = I.Workload("unaligned", T=301, H=16, E=E, k=8, R=1)
    logits = I.make_logits(wl)
    idx_ref, w_ref = oracle.route_topk(logits, wl.k)
    buf = torch.empty(wl.T * E + 1, dtype=torch.float32, device="cuda")
    view = buf[1:].view(wl.T, E)
    view.copy_(dev(logits))
    assert view.data_ptr() % 16 == 4
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    B.moe_route_topk(view, wl.k, idx, w)
    np.testing.assert_array_equal(host(idx), idx_ref)
    assert_weights(host(w), w_ref)


@pytest.mark.parametrize("E", [64, 128, 256])
@pytest.mark.parametrize("k", [1, 4, 8, 9])
def test_route_ties_and_concentrated_picks(E, k):
    """Many equal logits across and within lanes (ties go to the lower expert
    id), tokens whose k largest logits all fall in one lane's block of
    experts (that lane supplies every pick), all-equal rows, and k = 9 (past
    the sorted-list selection's k <= 8)."""
    rng = np.random.default_rng(E * 100 + k)
    T = 777
    logits = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    per_lane = E // 16
    for t in range(0, T, 7):      # one lane's block (start varies) dominates
        b = (t // 7) % 16 * per_lane
        logits[t, b:b + per_lane] += 20.0
    for t in range(3, T, 11):     # all equal
        logits[t] = 0.25
    for t in range(5, T, 13):     # equal maxima in two lanes' blocks
        logits[t, per_lane + 1] = logits[t, 3 * per_lane] = 30.0
    idx_ref, w_ref = oracle.route_topk(logits, k)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route_topk(dev(logits), k, idx, w)
    np.testing.assert_array_equal(host(idx), idx_ref)
    assert host(idx)[3].tolist() == list(range(k))
    assert_weights(host(w), w_ref)


def test_route_ties_and_signed_zero():
    rng = np.random.default_rng(0)
    T, E, k = 512, 64, 8
    logits = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)  # many ties
    logits[0] = 0.0
    logits[1] = 0.0
    logits[1, ::2] = -0.0
    logits[2] = 1.5
    idx_ref, w_ref = oracle.route_topk(logits, k)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route_topk(dev(logits), k, idx, w)
    np.testing.assert_array_equal(host(idx), idx_ref)
    assert host(idx)[1].tolist() == list(range(k))
    assert_weights(host(w), w_ref)


def _ulps(x, n):
    """x moved n float32 ulps up (n > 0) or down."""
    x = np.float32(x)
    for _ in range(abs(n)):
        x = np.nextafter(x, np.float32(np.inf if n > 0 else -np.inf), dtype=np.float32)
    return x


@pytest.mark.parametrize("E", [64, 128, 256])
@pytest.mark.parametrize("k", [1, 2, 8])
def test_route_near_ties(E, k):
    """Logits a few ulps apart where the order is decided: the router's fast
    selection compares keys that keep only the top 24 bits of the logit's
    order-preserving image, so picks within 256 ulps of each other (at the
    top, at the cut between the k-th and (k+1)-th pick, inside one lane's
    block of experts or across lanes) must be ordered exactly all the same;
    a pair straddling a 256-ulp boundary and near-ties below the cut are
    mixed in.  The kind changes every 4 tokens (one wavefront's tokens), so
    the waves of kinds 3-5 take the fast selection and the others redo
    theirs with full keys."""
    rng = np.random.default_rng(E * 10 + k)
    T = 640
    logits = rng.standard_normal((T, E)).astype(np.float32)
    per_lane = E // 16
    for t in range(T):
        kind = (t // 4) % 6
        a, b = rng.choice(E, size=2, replace=False)
        lo, hi = min(a, b), max(a, b)
        if kind == 0:    # top pick: the higher id is 1 ulp larger
            logits[t, lo] = 6.0
            logits[t, hi] = _ulps(6.0, 1)
        elif kind == 1:  # the k-th and (k+1)-th picks a few ulps apart
            logits[t, :] = np.minimum(logits[t], np.float32(1.0))
            big = rng.choice(E, size=k + 1, replace=False)
            logits[t, big] = 4.0 + np.arange(k + 1, dtype=np.float32)[::-1]
            hi_id = big.max()
            lo_id = big.min()
            logits[t, lo_id] = np.float32(2.5)
            logits[t, hi_id] = _ulps(2.5, 3)
        elif kind == 2:  # inside one lane's block: later expert 2 ulps larger
            base = rng.integers(16) * per_lane
            logits[t, base] = 7.0
            logits[t, base + per_lane - 1] = _ulps(7.0, 2)
        elif kind == 3:  # 1 ulp apart across a 256-ulp boundary of the image
            x = np.float32(np.frombuffer(np.uint32(0x40A000FF).tobytes(), np.float32)[0])
            logits[t, lo] = x
            logits[t, hi] = _ulps(x, 1)
        elif kind == 4:  # near-ties far below the cut
            logits[t, lo] = -5.0
            logits[t, hi] = _ulps(-5.0, 1)
        # kind 5: plain normal logits
    idx_ref, w_ref = oracle.route_topk(logits, k)
    for fused in (False, True):
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        if fused:
            lay = B.alloc_layout_chunks(T, T, E, k, 1, "cuda")
            B.moe_route_layout_chunks(dev(logits), k, 1, 0, None, idx, w, lay)
        else:
            B.moe_route_topk(dev(logits), k, idx, w)
        np.testing.assert_array_equal(host(idx), idx_ref)
        assert_weights(host(w), w_ref)


def _mixed_logits(rng, T, E):
    """Per token one of: normal; small integers (exact ties); a run of
    values 0-700 ulps above one base (crossing 256-ulp blocks of the
    router's 32-bit keys); negatives with +0 / -0; subnormals; magnitudes
    near 1e30 (most weights underflow to exactly 0); five experts tied at
    the top."""
    z = rng.standard_normal((T, E)).astype(np.float32)
    for t, kd in enumerate(rng.integers(0, 7, size=T)):
        if kd == 1:
            z[t] = rng.integers(-3, 4, size=E).astype(np.float32)
        elif kd == 2:
            base = np.float32(rng.choice([0.75, 3.0, -2.0, 40.0]))
            z[t] = (np.full(E, base).view(np.int32)
                    + rng.integers(0, 700, size=E).astype(np.int32)).view(np.float32)
        elif kd == 3:
            z[t] = -np.abs(z[t])
            m = rng.random(E) < 0.3
            z[t, m] = np.where(rng.random(m.sum()) < 0.5, np.float32(0.0), np.float32(-0.0))
        elif kd == 4:
            z[t] = (rng.standard_normal(E) * 1e-40).astype(np.float32)
        elif kd == 5:
            z[t] = (rng.standard_normal(E) * 1e30).astype(np.float32)
        elif kd == 6:
            z[t, rng.choice(E, size=min(E, 5), replace=False)] = np.float32(9.0)
    return z


@pytest.mark.parametrize("E,k", [(64, 8), (128, 1), (128, 8), (256, 4), (256, 8), (256, 16),
                                 (1000, 8)])
def test_route_mixed_ties_and_magnitudes(E, k):
    """Exact ties, ulp-close runs, signed zeros, subnormal and huge logits
    (weights that underflow to exactly 0) mixed token by token, so most
    wavefronts hold several kinds: ids bit-exact and weights within their
    bar (a zero reference weight must be zero) on the router and on the
    fused route + layout, whose weights equal the router's bit for bit."""
    rng = np.random.default_rng(E * 100 + k)
    T = 2000
    logits = _mixed_logits(rng, T, E)
    idx_ref, w_ref = oracle.route_topk(logits, k)
    assert k == 1 or (w_ref == 0).any()  # underflowed weights are exercised
    ws = []
    for fused in (False, True):
        print(f"route mixed E={E} k={k} fused={fused}", flush=True)
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        if fused:
            lay = B.alloc_layout_chunks(T, T, E, k, 1, "cuda")
            B.moe_route_layout_chunks(dev(logits), k, 1, 0, None, idx, w, lay)
        else:
            B.moe_route_topk(dev(logits), k, idx, w)
        np.testing.assert_array_equal(host(idx), idx_ref)
        assert_weights(host(w), w_ref)
        ws.append(host(w))
    np.testing.assert_array_equal(ws[0], ws[1])


# ------------------------------------------------------------------ layout
def gpu_layout(idx_np, E, R, cap):
    Tc, k = idx_np.shape
    lay = B.alloc_layout(Tc, E, k, R, "cuda")
    lay.pos.fill_(-7)
    lay.row_src.fill_(-7)
    B.moe_dispatch_layout(dev(idx_np), Tc, E, k, R, cap, lay)
    torch.cuda.synchronize()
    return lay


def assert_layout_equal(lay, ref, S):
    np.testing.assert_array_equal(host(lay.expert_counts), ref.expert_counts)
    np.testing.assert_array_equal(host(lay.expert_offsets), ref.expert_offsets)
    np.testing.assert_array_equal(host(lay.rank_counts), ref.rank_counts)
    np.testing.assert_array_equal(host(lay.rank_offsets), ref.rank_offsets)
    np.testing.assert_array_equal(host(lay.pos)[:S], ref.pos.ravel())
    np.testing.assert_array_equal(host(lay.row_src)[:S], ref.row_src)


LAYOUT_CASES = [
    # name, T, E, k, R, capacity, skew
    ("tiny", 256, 8, 2, 2, 0, None),
    ("one_token", 1, 8, 2, 2, 0, None),
    ("ragged", 1001, 37 * 2, 5, 2, 0, None),
    ("mid", 4096, 64, 8, 8, 0, None),
    ("dsv3_chunk_zipf", 4096, 256, 8, 32, 0, 1.1),
    ("cap_qwen_chunk", 4096, 128, 8, 16, 320, None),
    ("cap_tight_zipf", 3000, 64, 4, 8, 50, 1.5),
    ("E1024_k16", 2000, 1024, 16, 64, 0, None),
    ("large_chunk", 32768, 64, 8, 8, 0, None),
]


@pytest.mark.parametrize("name,T,E,k,R,cap,skew", LAYOUT_CASES, ids=[c[0] for c in LAYOUT_CASES])
def test_layout_parity(name, T, E, k, R, cap, skew):
    wl = I.Workload(name, T=T, H=16, E=E, k=k, R=R, zipf_s=skew)
    idx_np, _ = oracle.route_topk(I.make_logits(wl), k)
    ref = oracle.dispatch_layout(idx_np, E, R, cap)
    lay = gpu_layout(idx_np, E, R, cap)
    assert_layout_equal(lay, ref, T * k)


def test_layout_all_tokens_one_expert_capacity():
    """Every token's first choice is expert 0 (the extreme of skew)."""
    T, E, k, R, cap = 5000, 16, 2, 4, 700
    rng = np.random.default_rng(2)
    idx_np = np.zeros((T, k), dtype=np.int32)
    idx_np[:, 1] = rng.integers(1, E, size=T)
    ref = oracle.dispatch_layout(idx_np, E, R, cap)
    lay = gpu_layout(idx_np, E, R, cap)
    assert_layout_equal(lay, ref, T * k)


CHUNKED_CASES = [
    # name, T, chunk_tokens, E, k, R, capacity factor, skew
    ("dsv3_4chunks", 16384, 4096, 256, 8, 32, None, 1.1),
    ("ragged_last", 1001, 300, 64, 4, 8, None, None),
    ("qwen_cap", 32768, 4096, 128, 8, 16, 1.25, None),
    ("tight_cap_ragged", 5000, 1200, 32, 4, 4, 0.5, 1.5),
    ("one_chunk", 777, 4096, 16, 2, 4, None, None),
]


@pytest.mark.parametrize("name,T,Tc,E,k,R,cf,skew", CHUNKED_CASES, ids=[c[0] for c in CHUNKED_CASES])
def test_layout_chunks_parity(name, T, Tc, E, k, R, cf, skew):
    """One batched call equals one oracle layout per chunk (per-chunk
    capacities from a device array when a factor is given)."""
    wl = I.Workload(name, T=T, H=16, E=E, k=k, R=R, zipf_s=skew)
    idx_np, _ = oracle.route_topk(I.make_logits(wl), k)
    C = -(-T // Tc)
    bounds = [(c * Tc, min(T, (c + 1) * Tc)) for c in range(C)]
    caps = [oracle.capacity_for(t1 - t0, k, E, cf) for t0, t1 in bounds]
    lay = B.alloc_layout_chunks(T, Tc, E, k, R, "cuda")
    lay.pos.fill_(-7)
    lay.row_src.fill_(-7)
    cap_dev = torch.tensor(caps, dtype=torch.int32, device="cuda") if cf else None
    B.moe_dispatch_layout_chunks(dev(idx_np), T, E, k, R, 0, cap_dev, lay)
    torch.cuda.synchronize()
    pos, row_src = host(lay.pos), host(lay.row_src)
    for c, (t0, t1) in enumerate(bounds):
        ref = oracle.dispatch_layout(idx_np[t0:t1], E, R, caps[c])
        np.testing.assert_array_equal(host(lay.expert_counts[c]), ref.expert_counts)
        np.testing.assert_array_equal(host(lay.expert_offsets[c]), ref.expert_offsets)
        np.testing.assert_array_equal(host(lay.rank_counts[c]), ref.rank_counts)
        np.testing.assert_array_equal(host(lay.rank_offsets[c]), ref.rank_offsets)
        np.testing.assert_array_equal(pos[t0 * k:t1 * k], ref.pos.ravel())
        np.testing.assert_array_equal(row_src[t0 * k:t1 * k], ref.row_src)


def test_layout_empty_chunk():
    E, R, k = 8, 2, 2
    lay = B.alloc_layout(0, E, k, R, "cuda")
    lay.expert_counts.fill_(9)
    lay.expert_offsets.fill_(9)
    lay.rank_counts.fill_(9)
    lay.rank_offsets.fill_(9)
    B.moe_dispatch_layout(torch.empty(0, dtype=torch.int32, device="cuda"), 0, E, k, R, 0, lay)
    torch.cuda.synchronize()
    assert host(lay.expert_counts).tolist() == [0] * E
    assert host(lay.expert_offsets).tolist() == [0] * (E + 1)
    assert host(lay.rank_counts).tolist() == [0] * R
    assert host(lay.rank_offsets).tolist() == [0] * (R + 1)


# ------------------------------------------------------------------ pack / combine, one chunk
PC_CASES = [
    # name, T, H, E, k, R, cap, outliers
    ("tiny", 256, 512, 8, 2, 2, 0, 0.0),
    ("H16", 100, 16, 8, 3, 2, 0, 0.0),
    ("H_ragged", 77, 16 * 67, 16, 4, 4, 0, 0.05),
    ("H7168", 300, 7168, 256, 8, 32, 0, 0.01),
    ("H8192_cap", 257, 8192, 64, 8, 8, 20, 0.0),
    ("H20000", 40, 20000, 8, 2, 2, 0, 0.0),
]


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
@pytest.mark.parametrize("name,T,H,E,k,R,cap,outl", PC_CASES, ids=[c[0] for c in PC_CASES])
def test_pack_standin_combine_parity(name, T, H, E, k, R, cap, outl, quant):
    wl = I.Workload(name, T=T, H=H, E=E, k=k, R=R, outlier_frac=outl)
    x = I.make_hidden(wl)
    if quant == 2 and H % 32:
        # int4 records need H % 32 == 0: the ABI refuses before launching
        pos = torch.zeros(T * k, dtype=torch.int32, device="cuda")
        buf = torch.zeros((T * k, 2 * H), dtype=torch.uint8, device="cuda")
        sc = torch.zeros(T * k, dtype=torch.float32, device="cuda")
        with pytest.raises(B.MoeError) as ei:
            B.moe_dispatch_pack(dev(x), T, H, k, pos, 2, buf, sc)
        assert ei.value.status == 2  # MOE_ERR_SHAPE
        return
    if T > 5:
        x[3] = 0  # an all-zero row: scale 0, codes 0
    logits = I.make_logits(wl)
    idx_np, w_np = oracle.route_topk(logits, k)
    ref = oracle.dispatch_layout(idx_np, E, R, cap)
    N = ref.n_rows
    rb = row_bytes(H, quant)
    send_ref = oracle.dispatch_pack(x, ref.pos, quant, n_rows=N)
    ret_ref = oracle.expert_standin(send_ref, quant, ref.expert_offsets, H, quant)
    out_ref = oracle.combine(ret_ref, quant, ref.pos, w_np, H)
    out_nox_ref = oracle.combine(send_ref, quant, ref.pos, w_np, H)

    lay = gpu_layout(idx_np, E, R, cap)
    rows = T * k
    # +1: canary row (and canary scale) past the last row any slot can reach
    send = torch.full((rows + 1, rb), 0xAB, dtype=torch.uint8, device="cuda")
    send_s = torch.full((rows + 1,), -3.0, dtype=torch.float32, device="cuda")
    B.moe_dispatch_pack(dev(x), T, H, k, lay.pos, quant, send, send_s)
    ret = torch.full((rows + 1, rb), 0xCD, dtype=torch.uint8, device="cuda")
    ret_s = torch.full((rows + 1,), -5.0, dtype=torch.float32, device="cuda")
    HN.moe_expert_standin(send, send_s, quant, lay.expert_offsets, E, rows, H, quant, ret, ret_s)
    w = dev(w_np)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    out_nox = torch.empty((T, H), dtype=torch.int16, device="cuda")
    B.moe_combine(ret, ret_s, quant, lay.pos, w, T, H, k, out)
    B.moe_combine(send, send_s, quant, lay.pos, w, T, H, k, out_nox)
    torch.cuda.synchronize()
    s, ss = host(send), host(send_s)
    compare_records(join_records(s[:N], ss[:N], H, quant), send_ref, H, quant, f"{name} pack")
    assert (s[N:] == 0xAB).all(), "pack wrote rows no slot points to"
    r, rs = host(ret), host(ret_s)
    compare_records(join_records(r[:N], rs[:N], H, quant), ret_ref, H, quant, f"{name} stand-in")
    assert (r[N:] == 0xCD).all()
    if quant:
        assert (ss[N:] == -3.0).all() and (rs[N:] == -5.0).all(), "scales written past N"
    assert_out_close(host(out), out_ref, f"{name} combine(stand-in)")
    assert_out_close(host(out_nox), out_nox_ref, f"{name} combine(identity)")


def _extreme_rows(rng, T, H):
    """bf16 hidden rows, one kind per token: ordinary; all zero with signed
    zeros; a single element of magnitude 1-2; subnormals only; magnitudes
    near the bf16 maximum; one maximal outlier among ordinary values; a
    constant row.  All finite."""
    x = I.make_hidden(I.Workload("x", T=T, H=H, E=8, k=1, R=1, seed=int(rng.integers(1 << 30))))
    for t, kd in enumerate(rng.integers(0, 8, size=T)):
        sign = rng.integers(0, 2, size=H).astype(np.uint16) << 15
        if kd == 1:
            x[t] = sign
        elif kd == 2:
            x[t] = 0
            x[t, rng.integers(H)] = 0x3F80 | int(rng.integers(0, 0x80)) | (int(rng.integers(0, 2)) << 15)
        elif kd == 3:
            x[t] = rng.integers(1, 0x80, size=H).astype(np.uint16) | sign
        elif kd == 4:
            x[t] = rng.integers(0x7F00, 0x7F80, size=H).astype(np.uint16) | sign
        elif kd == 5:
            x[t, rng.integers(H)] = 0x7F7F
        elif kd == 6:
            x[t] = x[t, 0]
    assert np.isfinite(I.bf16_bits_to_f32(x)).all()
    return x


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
def test_pack_combine_extreme_rows(quant):
    """Rows whose scale underflows (subnormal-only rows, whose fp32 scale is
    itself subnormal), rows near the bf16 maximum, single-element, constant
    and signed-zero rows: the pack's rows and scales to their bar (codes
    were bit-exact in 232 random draws of these kinds) and the combine of
    the rows straight back (no expert) within the output bar."""
    rng = np.random.default_rng(40 + quant)
    T, H, E, k = 700, 1056, 64, 8
    x = _extreme_rows(rng, T, H)
    logits = I.make_logits(I.Workload("l", T=T, H=H, E=E, k=k, R=1, seed=3))
    idx_np, w_np = oracle.route_topk(logits, k)
    ref = oracle.dispatch_layout(idx_np, E, 1, 0)
    N = ref.n_rows
    send_ref = oracle.dispatch_pack(x, ref.pos, quant, n_rows=N)
    out_ref = oracle.combine(send_ref, quant, ref.pos, w_np, H)
    lay = gpu_layout(idx_np, E, 1, 0)
    send = torch.zeros((T * k, row_bytes(H, quant)), dtype=torch.uint8, device="cuda")
    send_s = torch.zeros(T * k, dtype=torch.float32, device="cuda")
    print(f"extreme rows q{quant}", flush=True)
    B.moe_dispatch_pack(dev(x), T, H, k, lay.pos, quant, send, send_s)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    B.moe_combine(send, send_s, quant, lay.pos, dev(w_np), T, H, k, out)
    torch.cuda.synchronize()
    compare_records(join_records(host(send)[:N], host(send_s)[:N], H, quant), send_ref, H, quant,
                    f"extreme rows q{quant} pack")
    assert_out_close(host(out), out_ref, f"extreme rows q{quant} combine")


def test_k1_roundtrip_identity_bitwise():
    """k = 1, bf16, no expert: permute then unpermute returns x bit for bit."""
    wl = I.Workload("k1", T=999, H=1024, E=16, k=1, R=4)
    x = I.make_hidden(wl)
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=3)
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    path.run(dev(I.make_logits(wl)), dev(x), out, quant=0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), x)


# ------------------------------------------------------------------ whole layers
def run_gpu_layer(wl, logits, x, quant, chunks, streams=1, standin=False, ring=None, cap_f=None):
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=chunks, streams=streams,
                             ring=ring or chunks, standin=standin)
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    path.run(dev(logits), dev(x), out, quant=quant, capacity_factor=cap_f)
    torch.cuda.synchronize()
    return path, out


@pytest.mark.parametrize("chunks", [1, 4])
def test_tiny_layer_end_to_end(chunks):
    """256 tokens, H=512, E=8, k=2, R=2, bf16, stand-in expert x*(1+e/8)."""
    wl = I.WORKLOADS["tiny"]
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    ref = oracle.run_layer(logits, x, wl.E, wl.k, wl.R, chunks=chunks, quant=0, standin=True)
    path, out = run_gpu_layer(wl, logits, x, 0, chunks, standin=True)
    np.testing.assert_array_equal(host(path.idx), ref.idx)
    assert_weights(host(path.w), ref.w)
    for c, (t0, t1) in enumerate(D.chunk_ranges(wl.T, chunks)):
        st = path.chunk_state(c)
        assert_layout_equal(st.layout, ref.layouts[c], (t1 - t0) * wl.k)
        N = ref.layouts[c].n_rows
        np.testing.assert_array_equal(host_records(st.send, None, N, wl.H, 0), ref.sends[c])
        np.testing.assert_array_equal(host_records(st.ret, None, N, wl.H, 0), ref.rets[c])
    assert_out_close(host(out), ref.out, "tiny")


def test_mid_int4_layer_end_to_end():
    """T=4096, H=4096, E=64, k=8, R=8, int4 both ways, stand-in experts,
    two chunks: every kept row and scale and every output against the oracle."""
    wl = I.WORKLOADS["mid"]
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    ref = oracle.run_layer(logits, x, wl.E, wl.k, wl.R, chunks=2, quant=2, standin=True,
                           workers=8)
    path, out = run_gpu_layer(wl, logits, x, 2, 2, standin=True)
    for c in range(2):
        st = path.chunk_state(c)
        N = ref.layouts[c].n_rows
        compare_records(host_records(st.send, st.send_scales, N, wl.H, 2), ref.sends[c], wl.H, 2,
                        "mid int4 pack")
        compare_records(host_records(st.ret, st.ret_scales, N, wl.H, 2), ref.rets[c], wl.H, 2,
                        "mid int4 stand-in")
    assert_out_close(host(out), ref.out, "mid int4")


def test_mid_int8_layer_end_to_end():
    """T=4096, H=4096, E=64, k=8, R=8, int8 both ways, one chunk."""
    wl = I.WORKLOADS["mid"]
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    ref = oracle.run_layer(logits, x, wl.E, wl.k, wl.R, chunks=1, quant=1, standin=True)
    path, out = run_gpu_layer(wl, logits, x, 1, 1, standin=True)
    np.testing.assert_array_equal(host(path.idx), ref.idx)
    st = path.chunk_state(0)
    assert_layout_equal(st.layout, ref.layouts[0], wl.T * wl.k)
    N = ref.layouts[0].n_rows
    compare_records(host_records(st.send, st.send_scales, N, wl.H, 1), ref.sends[0], wl.H, 1,
                    "mid pack")
    compare_records(host_records(st.ret, st.ret_scales, N, wl.H, 1), ref.rets[0], wl.H, 1,
                    "mid stand-in")
    assert_out_close(host(out), ref.out, "mid int8")


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
def test_dsv3_full_size_sampled(quant):
    """T=16384, H=7168, E=256, k=8, R=32, Zipf-skewed routing, 1% x50 rows,
    in the chunk count the benchmark times for the payload (8 bf16, 4 int8
    and int4):
    routing and layouts compared in full, send rows and outputs on samples
    the oracle computes one by one."""
    wl = I.WORKLOADS["dsv3"]
    wl = wl.with_(chunks=D.resolve_chunks(wl, quant))
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    idx_ref, w_ref = oracle.route_topk(logits, wl.k)
    path, out = run_gpu_layer(wl, logits, x, quant, wl.chunks)  # one staging buffer per chunk
    np.testing.assert_array_equal(host(path.idx), idx_ref)
    assert_weights(host(path.w), w_ref)
    rng = np.random.default_rng(5)
    outl = set(I.outlier_rows(wl).tolist())
    out_h = host(out)
    for c, (t0, t1) in enumerate(D.chunk_ranges(wl.T, wl.chunks)):
        lref = oracle.dispatch_layout(idx_ref[t0:t1], wl.E, wl.R)
        st = path.chunk_state(c)
        assert_layout_equal(st.layout, lref, (t1 - t0) * wl.k)
        rows = rng.choice(lref.n_rows, size=256, replace=False)
        toks = t0 + lref.row_src[rows] // wl.k
        got = sampled_records(st.send, st.send_scales, lref.n_rows, rows, wl.H, quant)
        pos_one = np.arange(len(rows), dtype=np.int32)[:, None]
        want = oracle.dispatch_pack(x[toks], pos_one, quant)
        compare_records(got, want, wl.H, quant, f"dsv3 chunk {c} pack")
    # outputs: sampled tokens including outlier rows
    sample = np.unique(np.concatenate([rng.choice(wl.T, 400, replace=False), sorted(outl)[:40]]))
    want = np.stack([oracle.roundtrip_token(x[t], np.zeros(wl.k, np.int32), w_ref[t], quant)
                     for t in sample])
    assert_out_close(out_h[sample], want, "dsv3 out")


def test_stream_modes_match_one_stream_bitwise():
    wl = I.Workload("s2", T=4096, H=1024, E=64, k=8, R=8)
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    _, o1 = run_gpu_layer(wl, logits, x, 1, 8, streams=1, standin=True, ring=2)
    _, o2 = run_gpu_layer(wl, logits, x, 1, 8, streams=2, standin=True, ring=2)
    _, o3 = run_gpu_layer(wl, logits, x, 1, 8, streams=2, standin=True, ring=2)
    _, o4 = run_gpu_layer(wl, logits, x, 1, 8, streams=3, standin=True, ring=2)
    np.testing.assert_array_equal(host(o1), host(o2))
    np.testing.assert_array_equal(host(o2), host(o3))
    np.testing.assert_array_equal(host(o1), host(o4))


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_two_streams_layouts_equal_one_stream(fused):
    """Two streams route chunk 0 on the caller's stream (its own workspace)
    while the control stream routes the other chunks: ids, weights, every
    chunk's layout (capacity factor 1.25, so slots are dropped per chunk) and
    the output equal the one-stream fused path's bit for bit, over two calls
    in a row on the same driver (the second with other inputs)."""
    wl = I.Workload("s2cap", T=5000, H=512, E=64, k=8, R=8, seed=5, zipf_s=1.1)
    wl2 = wl.with_(seed=6)
    one = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=5, streams=1, ring=2)
    two = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=5, streams=2, ring=2,
                            fused=fused)
    for w in (wl, wl2):
        print(f"two streams fused={fused} seed={w.seed}", flush=True)
        x, lg = dev(I.make_hidden(w)), dev(I.make_logits(w))
        o1 = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
        o2 = torch.empty_like(o1)
        one.run(lg, x, o1, quant=1, capacity_factor=1.25)
        two.run(lg, x, o2, quant=1, capacity_factor=1.25)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(two.idx), host(one.idx))
        np.testing.assert_array_equal(host(two.w), host(one.w))
        for c in range(5):
            a, b = one.chunk_state(c).layout, two.chunk_state(c).layout
            for name in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets"):
                np.testing.assert_array_equal(host(getattr(b, name)), host(getattr(a, name)),
                                              err_msg=f"chunk {c} {name}")
            n = a.pos.numel()
            np.testing.assert_array_equal(host(b.pos)[:n], host(a.pos)[:n])
            np.testing.assert_array_equal(host(b.row_src)[:n], host(a.row_src)[:n])
        assert int((host(one.chunk_state(0).layout.pos) < 0).sum()) > 0  # drops happen
        np.testing.assert_array_equal(host(o2), host(o1))


def test_chunk_count_does_not_change_output():
    wl = I.Workload("ch", T=2048, H=512, E=32, k=4, R=4)
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    outs = [host(run_gpu_layer(wl, logits, x, 0, c, standin=True)[1]) for c in (1, 4, 8)]
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_qwen3_stack_layerwise():
    """4-layer stack T=32768, H=2048, E=128, k=8, R=16, 8 chunks on 2 streams,
    capacity factor 1.25 (drops by token id), int8 on the middle layers.  Each
    layer's GPU input is the oracle chain's input for that layer."""
    wl = I.WORKLOADS["qwen3"]
    x = I.make_hidden(wl)
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=wl.chunks, streams=2,
                             ring=2, standin=True)
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    cur = x
    for layer, q in enumerate(wl.quant):
        logits = I.make_logits(wl, layer)
        ref = oracle.run_layer(logits, cur, wl.E, wl.k, wl.R, chunks=wl.chunks, quant=q,
                               capacity_factor=wl.capacity_factor, standin=True,
                               keep_buffers=False, workers=8)
        path.run(dev(logits), dev(cur), out, quant=q, capacity_factor=wl.capacity_factor)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(path.idx), ref.idx)
        dropped = sum(int((l.pos < 0).sum()) for l in ref.layouts)
        assert_out_close(host(out), ref.out, f"qwen3 layer {layer} (int8={q}, dropped {dropped})")
        cur = ref.out


@pytest.fixture(scope="module")
def large_inputs():
    wl = I.WORKLOADS["large"]
    x = I.make_hidden(wl)
    logits = I.make_logits(wl)
    idx_ref, w_ref = oracle.route_topk(logits, wl.k)
    return wl, x, logits, idx_ref, w_ref


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
def test_large_full_size_sampled(large_inputs, quant):
    """T=131072, H=8192, E=64, k=8, R=8 in 4 chunks (2^34 bytes per direction
    for bf16): routing and every chunk's layout compared in full, send rows
    and outputs on samples the oracle computes one by one."""
    wl, x, logits, idx_ref, w_ref = large_inputs
    path, out = run_gpu_layer(wl, logits, x, quant, wl.chunks, ring=2)
    np.testing.assert_array_equal(host(path.idx), idx_ref)
    assert_weights(host(path.w), w_ref)
    rng = np.random.default_rng(7)
    for c, (t0, t1) in enumerate(D.chunk_ranges(wl.T, wl.chunks)):
        lref = oracle.dispatch_layout(idx_ref[t0:t1], wl.E, wl.R)
        assert_layout_equal(path.chunk_state(c).layout, lref, (t1 - t0) * wl.k)
    # the staging ring holds the last two chunks' send buffers
    for c in (wl.chunks - 2, wl.chunks - 1):
        t0, t1 = D.chunk_ranges(wl.T, wl.chunks)[c]
        lref = oracle.dispatch_layout(idx_ref[t0:t1], wl.E, wl.R)
        rows = rng.choice(lref.n_rows, size=128, replace=False)
        toks = t0 + lref.row_src[rows] // wl.k
        st = path.chunk_state(c)
        got = sampled_records(st.send, st.send_scales, lref.n_rows, rows, wl.H, quant)
        want = oracle.dispatch_pack(x[toks], np.arange(len(rows), dtype=np.int32)[:, None], quant)
        compare_records(got, want, wl.H, quant, f"large chunk {c} pack")
    sample = rng.choice(wl.T, 300, replace=False)
    want = np.stack([oracle.roundtrip_token(x[t], np.zeros(wl.k, np.int32), w_ref[t], quant)
                     for t in sample])
    assert_out_close(host(out[torch.from_numpy(sample).cuda()]), want, "large out")
    del path, out
    torch.cuda.empty_cache()
