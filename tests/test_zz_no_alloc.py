"""moe_route_layout_chunks_noalloc (histogram scratch in the library's static
device buffer) against moe_route_layout_chunks (caller's workspace), through
the C ABI: every output bit for bit, over consecutive calls that shrink, so
that the previous call's scratch contents cannot leak into the next."""
import numpy as np
import pytest
import torch

from combine_fp32_router_amd import binding as B
from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I

pytestmark = pytest.mark.gpu


def _both(logits, k, R, chunks, capacity_factor=None):
    T, E = logits.shape
    Tc = -(-T // chunks) if T else 1
    caps = None
    if capacity_factor:
        caps = torch.tensor([D.chunk_capacity(t1 - t0, k, E, capacity_factor)
                             for t0, t1 in D.chunk_ranges(T, chunks)],
                            dtype=torch.int32, device="cuda")
    res = []
    for fn in (B.moe_route_layout_chunks, B.moe_route_layout_chunks_noalloc):
        lay = B.alloc_layout_chunks(T, Tc, E, k, R, "cuda", chunks)
        # poison every output so that an entry the call does not write shows up
        for t in (lay.expert_counts, lay.expert_offsets, lay.rank_counts, lay.rank_offsets,
                  lay.pos, lay.row_src):
            t.fill_(-7)
        idx = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((max(T, 1), k), -7.0, dtype=torch.float32, device="cuda")
        fn(logits, k, R, 0, caps, idx, w, lay)
        res.append((idx, w, lay))
    torch.cuda.synchronize()
    return res


def _assert_same(ref, got, what):
    (i0, w0, l0), (i1, w1, l1) = ref, got
    assert torch.equal(i0, i1), f"{what}: topk_idx"
    assert torch.equal(w0.view(torch.int32), w1.view(torch.int32)), f"{what}: topk_w"
    for name in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pos",
                 "row_src"):
        assert torch.equal(getattr(l0, name), getattr(l1, name)), f"{what}: {name}"


CASES = [
    # (workload, T, E, k, R, chunks, capacity factor): each smaller than the last
    ("dsv3", 16384, 256, 8, 32, 8, None),      # fused router, 256 KiB of scratch
    ("mid", 4096, 64, 8, 8, 1, 1.0),           # fused, one chunk, capacity drops
    ("ragged", 1000, 36, 6, 4, 3, 1.25),       # k = 6: separate route + layout passes
    ("empty", 0, 64, 8, 8, 1, None),           # T = 0: zero counts and offsets
]


def test_noalloc_matches_workspace_call_over_shrinking_calls():
    for name, T, E, k, R, chunks, cf in CASES:
        print(f"noalloc case {name}: T={T} E={E} k={k} R={R} chunks={chunks} cf={cf}",
              flush=True)
        if name in I.WORKLOADS:
            wl = I.WORKLOADS[name]
            assert (wl.T, wl.E, wl.k, wl.R) == (T, E, k, R)
            logits = I.make_logits(wl)
        else:
            logits = np.random.default_rng(3).standard_normal((T, E)).astype(np.float32)
        ref, got = _both(torch.from_numpy(logits).cuda(), k, R, chunks, cf)
        _assert_same(ref, got, name)
        if T:
            n_rows = ref[2].expert_offsets[:, -1].cpu().numpy()
            assert n_rows.sum() <= T * k and n_rows.min() > 0
        else:
            assert int(ref[2].expert_offsets.abs().sum()) == 0


def test_noalloc_twice_in_a_row_on_one_stream():
    """Two calls queued back to back on one stream (the second smaller),
    synchronised only at the end: each equals its workspace counterpart."""
    wl_a, wl_b = I.WORKLOADS["dsv3"], I.WORKLOADS["mid"]
    outs = []
    for wl, chunks in ((wl_a, 8), (wl_b, 1)):
        logits = torch.from_numpy(I.make_logits(wl)).cuda()
        Tc = -(-wl.T // chunks)
        lay = B.alloc_layout_chunks(wl.T, Tc, wl.E, wl.k, wl.R, "cuda", chunks)
        idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        B.moe_route_layout_chunks_noalloc(logits, wl.k, wl.R, 0, None, idx, w, lay)
        outs.append((wl, chunks, logits, (idx, w, lay)))
    torch.cuda.synchronize()
    for wl, chunks, logits, got in outs:
        ref = _both(logits, wl.k, wl.R, chunks)[0]
        _assert_same(ref, got, f"{wl.name} queued")
