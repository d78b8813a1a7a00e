"""GPU parity of the fused router + layout call (moe_route_layout_chunks):
every output equals the oracle's route followed by one oracle layout per
chunk (ids, counts, offsets, pos, row_src bit-exact; weights 1e-6
relative), and equals the two separate GPU calls bit for bit.  Cases cover
the fused tiling (k dividing the layout tile into whole router groups, for
64-token and 16-token groups, ragged last chunks, capacity drops) and the
fallbacks (k = 6: groups straddle tiles; a histogram past the fold
budget)."""
import numpy as np
import pytest
import torch

import oracle
from combine_fp32_router_amd import binding as B
from combine_fp32_router_amd import inputs as I
from gpu_util import assert_weights, dev, host

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, Tc, E, k, R, capacity factor, zipf, fused tiling expected
    ("dsv3_8chunks", 16384, 2048, 256, 8, 32, None, 1.1, True),
    ("mid_1chunk", 4096, 4096, 64, 8, 8, None, None, True),
    ("ragged_chunks", 1001, 300, 64, 4, 8, None, None, True),
    ("k1", 500, 128, 64, 1, 8, None, None, True),
    ("E1024_k16", 333, 100, 1024, 16, 8, None, None, True),
    ("E512_k2", 777, 256, 512, 2, 4, None, None, True),
    ("qwen_cap", 4096, 512, 128, 8, 16, 1.25, None, True),
    ("k6_fallback", 700, 256, 200, 6, 5, None, None, False),
    ("one_token", 1, 1, 8, 2, 2, None, None, True),
    ("large_chunk_fused", 65536, 32768, 64, 8, 8, None, None, True),     # 512 rows x 64 <= 64K
    ("large_chunk_unfused", 65536, 32768, 256, 8, 32, None, None, False),  # 512 x 256 > 64K
]


@pytest.mark.parametrize("name,T,Tc,E,k,R,cf,skew,fusable", CASES, ids=[c[0] for c in CASES])
def test_route_layout_fused_parity(name, T, Tc, E, k, R, cf, skew, fusable):
    wl = I.Workload(name, T=T, H=16, E=E, k=k, R=R, zipf_s=skew)
    logits = I.make_logits(wl)
    if cf:
        logits = logits.copy()
        logits[:, 3] += 2.0                      # an overloaded expert: drops happen
    idx_ref, w_ref = oracle.route_topk(logits, k)
    C = -(-T // Tc)
    bounds = [(c * Tc, min(T, (c + 1) * Tc)) for c in range(C)]
    caps = [oracle.capacity_for(t1 - t0, k, E, cf) for t0, t1 in bounds]
    cap_dev = torch.tensor(caps, dtype=torch.int32, device="cuda") if cf else None
    ws_fused = B.route_layout_workspace_bytes(T, Tc, E, k, R)
    ws_plain = B.layout_chunks_workspace_bytes(T, Tc, E, k, R)
    assert (ws_fused != ws_plain) == fusable or T == 1

    lg = dev(logits)
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    lay = B.alloc_layout_chunks(T, Tc, E, k, R, "cuda")
    lay.pos.fill_(-7)
    lay.row_src.fill_(-7)
    B.moe_route_layout_chunks(lg, k, R, 0, cap_dev, idx, w, lay)
    # the separate calls
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    lay2 = B.alloc_layout_chunks(T, Tc, E, k, R, "cuda")
    B.moe_route_topk(lg, k, idx2, w2)
    B.moe_dispatch_layout_chunks(idx2, T, E, k, R, 0, cap_dev, lay2)
    torch.cuda.synchronize()

    np.testing.assert_array_equal(host(idx), idx_ref)
    assert_weights(host(w), w_ref)
    pos, row_src = host(lay.pos), host(lay.row_src)
    dropped = 0
    for c, (t0, t1) in enumerate(bounds):
        ref = oracle.dispatch_layout(idx_ref[t0:t1], E, R, caps[c])
        np.testing.assert_array_equal(host(lay.expert_counts[c]), ref.expert_counts)
        np.testing.assert_array_equal(host(lay.expert_offsets[c]), ref.expert_offsets)
        np.testing.assert_array_equal(host(lay.rank_counts[c]), ref.rank_counts)
        np.testing.assert_array_equal(host(lay.rank_offsets[c]), ref.rank_offsets)
        np.testing.assert_array_equal(pos[t0 * k:t1 * k], ref.pos.ravel())
        np.testing.assert_array_equal(row_src[t0 * k:t1 * k], ref.row_src)
        dropped += int((ref.pos < 0).sum())
    if cf:
        assert dropped > 0
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    for a, b in zip(lay[:6], lay2[:6]):
        assert torch.equal(a[:C], b[:C]) if a.dim() == 2 else torch.equal(a, b)


def test_route_layout_empty_batch():
    E, R, k = 8, 2, 2
    lay = B.alloc_layout_chunks(0, 1, E, k, R, "cuda")
    lay.expert_counts.fill_(9)
    lay.expert_offsets.fill_(9)
    lay.rank_counts.fill_(9)
    lay.rank_offsets.fill_(9)
    lg = torch.empty((0, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((0, k), dtype=torch.int32, device="cuda")
    w = torch.empty((0, k), dtype=torch.float32, device="cuda")
    B.moe_route_layout_chunks(lg, k, R, 0, None, idx, w, lay)
    torch.cuda.synchronize()
    assert (host(lay.expert_counts[0]) == 0).all()
    assert (host(lay.expert_offsets[0]) == 0).all()
    assert (host(lay.rank_counts[0]) == 0).all()
    assert (host(lay.rank_offsets[0]) == 0).all()
