"""Pins for the oracle's dispatch layout (O2): histogram, scans, rank
blocks, stable pos/row_src, capacity drops."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(int, ln.split())) for ln in f if ln.strip() and not ln.startswith("#")]


def _random_idx(rng, Tc, E, k):
    """Distinct experts per token, as top-k produces."""
    return np.argsort(rng.random((Tc, E)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("Tc,E,k,R", [(1, 8, 2, 2), (257, 8, 2, 2), (1000, 64, 8, 8),
                                      (333, 256, 8, 32), (64, 12, 3, 4)])
def test_permutation_is_numpy_stable_argsort(Tc, E, k, R):
    rng = np.random.default_rng(Tc + E)
    idx = _random_idx(rng, Tc, E, k)
    lay = oracle.dispatch_layout(idx, E, R)
    flat = idx.ravel()
    # histogram and exclusive scan
    np.testing.assert_array_equal(lay.expert_counts, np.bincount(flat, minlength=E))
    assert lay.expert_counts.sum() == Tc * k
    np.testing.assert_array_equal(lay.expert_offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    # rows ordered by (expert, slot): numpy's stable argsort of the slot experts
    np.testing.assert_array_equal(lay.row_src, np.argsort(flat, kind="stable"))
    # pos is the inverse permutation: a bijection slots -> [0, N)
    inv = np.empty_like(lay.row_src)
    inv[lay.row_src] = np.arange(Tc * k)
    np.testing.assert_array_equal(lay.pos.ravel(), inv)
    # contiguous rank blocks of E/R experts; at most R non-empty blocks
    per = E // R
    np.testing.assert_array_equal(lay.rank_offsets[:-1], lay.expert_offsets[::per][:R])
    assert lay.rank_offsets[-1] == Tc * k
    np.testing.assert_array_equal(lay.rank_counts, np.diff(lay.rank_offsets))
    rank_of_row = flat[lay.row_src] // per
    assert np.all(np.diff(rank_of_row) >= 0)


def test_ep_placement_example_from_page():
    """Communication-wall page, EP=8 example: experts 5, 18, 41, 63 of 64 land
    on GPUs 0, 2, 5, 7."""
    rows = _rows("commwall_ep_placement.txt")
    E, R = rows[0]
    toks = rows[1:]
    idx = np.array([[e] for _, e, _ in toks], dtype=np.int32)
    lay = oracle.dispatch_layout(idx, E, R)
    want = np.zeros(R, dtype=np.int32)
    for _, _, g in toks:
        want[g] += 1
    np.testing.assert_array_equal(lay.rank_counts, want)
    for s, (_, e, g) in enumerate(toks):
        p = lay.pos[s, 0]
        assert lay.rank_offsets[g] <= p < lay.rank_offsets[g + 1]


def test_flat_sendcounts_example_from_page():
    """NCCL EP page s3.3: segment r of the flat buffer starts at the sum of
    the earlier ranks' counts, zero-length segments included.  One row per
    count unit (1 KiB rows), E = R = 8, k = 1."""
    counts = np.array(_rows("ncclep_sendcounts.txt")[0]) // 1024
    idx = np.repeat(np.arange(8, dtype=np.int32), counts)[:, None]
    idx = np.ascontiguousarray(np.random.default_rng(0).permutation(idx))
    lay = oracle.dispatch_layout(idx, 8, 8)
    np.testing.assert_array_equal(lay.rank_counts, counts)
    np.testing.assert_array_equal(lay.rank_offsets, [0, 0, 1024, 1536, 3584, 3584, 3584, 3584, 3584])


def test_capacity_keeps_lowest_token_ids():
    """Every token's first choice is expert 0; with capacity c exactly the
    first c tokens keep that slot, the rest are dropped (-1), and surviving
    rows are still ordered by token."""
    Tc, E, k, R, cap = 100, 8, 2, 2, 30
    rng = np.random.default_rng(4)
    idx = np.zeros((Tc, k), dtype=np.int32)
    idx[:, 1] = rng.integers(1, E, size=Tc)
    lay = oracle.dispatch_layout(idx, E, R, capacity=cap)
    assert lay.expert_counts[0] == Tc
    assert lay.expert_offsets[1] == cap
    assert (lay.pos[:cap, 0] >= 0).all() and (lay.pos[cap:, 0] == -1).all()
    np.testing.assert_array_equal(lay.pos[:cap, 0], np.arange(cap))
    N = lay.n_rows
    assert N == cap + Tc - np.maximum(np.bincount(idx[:, 1], minlength=E)[1:] - cap, 0).sum()
    assert (lay.row_src[N:] == -1).all()
    kept = lay.row_src[:N]
    assert (kept >= 0).all()
    np.testing.assert_array_equal(lay.pos.ravel()[kept], np.arange(N))
    # dropped slots are exactly the ones not referenced by row_src
    assert (lay.pos.ravel() == -1).sum() == Tc * k - N


def test_capacity_general_against_brute_force():
    """Capacity per expert: kept slots are the first `cap` slots of each
    expert in slot order (brute force with a Python counter)."""
    rng = np.random.default_rng(8)
    for trial in range(5):
        Tc, E, k, R = 200, 16, 4, 4
        # skewed: expert ids drawn from a steep distribution
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(Tc)]).astype(np.int32)
        cap = int(rng.integers(1, 60))
        lay = oracle.dispatch_layout(idx, E, R, capacity=cap)
        seen = {}
        kept_slots = []
        for s, e in enumerate(idx.ravel().tolist()):
            seen[e] = seen.get(e, 0) + 1
            if seen[e] <= cap:
                kept_slots.append((e, s))
        kept_slots.sort()
        np.testing.assert_array_equal(lay.row_src[:len(kept_slots)], [s for _, s in kept_slots])
        assert lay.n_rows == len(kept_slots)


def test_empty_chunk():
    idx = np.zeros((0, 2), dtype=np.int32)
    lay = oracle.dispatch_layout(idx, 8, 2)
    assert lay.n_rows == 0 and lay.expert_counts.sum() == 0
    assert lay.rank_offsets.tolist() == [0, 0, 0]


def test_rejects_bad_shapes():
    idx = np.zeros((4, 2), dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.dispatch_layout(idx, 8, 3)  # E % R != 0
    with pytest.raises(ValueError):
        oracle.dispatch_layout(idx + 9, 8, 2)  # expert id out of range
