"""Pins of the receiver-side oracle (recv_layout, exchange, regroup,
run_ep_layer) against facts that do not come from the oracle itself: the
8-rank receive-count example of the NCCL EP article (s3.3), the count-matrix
transpose, the single-source layout of the whole batch (a sort by expert is
stable, so regrouping R consecutive shards by expert then source equals
sorting the whole batch by expert), brute force on tagged rows, inverse
round trips, and the chunked layer."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(int, ln.split())) for ln in f if ln.strip() and not ln.startswith("#")]


def _random_idx(rng, T, E, k):
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def _tagged_rows(T, H):
    """bf16 bit patterns whose first two elements spell the token id."""
    x = np.zeros((T, H), dtype=np.uint16)
    x[:, 0] = np.arange(T) & 0xFFFF
    x[:, 1] = np.arange(T) >> 16
    x[:, 2:] = np.random.default_rng(1).integers(0, 0x7F00, size=(T, H - 2), dtype=np.uint16)
    return x


def _shard_layouts(idx, E, R, cap=0):
    bounds = oracle.chunk_bounds(idx.shape[0], R)
    lays = [oracle.dispatch_layout(idx[t0:t1], E, R, cap) for t0, t1 in bounds]
    return bounds, lays, np.stack([l.expert_offsets for l in lays])


def _send_buffer(x, bounds, lays, k, quant=0):
    source_rows = (bounds[0][1] - bounds[0][0]) * k
    send = np.zeros((len(bounds) * source_rows, oracle.record_bytes(x.shape[1], quant)), np.uint8)
    for s, ((t0, t1), lay) in enumerate(zip(bounds, lays)):
        if t1 > t0:
            send[s * source_rows:s * source_rows + (t1 - t0) * k] = oracle.dispatch_pack(
                x[t0:t1], lay.pos, quant)
    return send, source_rows


def test_ncclep_receive_counts_example():
    """Rank 0 of the article's 8-rank example receives 2 MiB, 1 MiB, 512 KiB
    and 1 MiB from ranks 4..7; its flat receive buffer holds those segments
    at 0, 2 MiB, 3 MiB and 3.5 MiB and ends at 4.5 MiB (units of 1 KiB rows
    below, one expert per rank)."""
    recvcounts = np.array(_rows("ncclep_recvcounts.txt")[0]) // 1024
    R = E = 8
    rng = np.random.default_rng(0)
    kept = rng.integers(0, 50, size=(R, E))
    kept[:, 0] = recvcounts            # what each source sends to rank 0's expert
    so = np.zeros((R, E + 1), dtype=np.int32)
    so[:, 1:] = np.cumsum(kept, axis=1)
    rl = oracle.recv_layout(so, R)
    np.testing.assert_array_equal(rl.recv_offsets[0], [0, 0, 0, 0, 0, 2048, 3072, 3584, 4608])
    assert rl.recv_offsets[1, 0] == 4608


def test_count_matrix_transpose():
    """Receiver r's segment from source s has source s's rank_counts[r] rows."""
    T, E, k, R = 600, 32, 4, 8
    idx = _random_idx(np.random.default_rng(2), T, E, k)
    bounds, lays, so = _shard_layouts(idx, E, R)
    rl = oracle.recv_layout(so, R)
    sizes = np.diff(rl.recv_offsets, axis=1)                  # [r, s]
    counts = np.stack([l.rank_counts for l in lays])          # [s, r]
    np.testing.assert_array_equal(sizes, counts.T)
    np.testing.assert_array_equal(rl.recv_offsets[1:, 0], rl.recv_offsets[:-1, R])


@pytest.mark.parametrize("R,E", [(4, 16), (8, 64), (1, 8), (8, 8)])
def test_grouped_equals_single_source_layout(R, E):
    """Capacity off: regrouping R shards by expert reproduces the one-source
    dispatch of the whole batch, row for row and offset for offset."""
    T, H, k = 512, 32, 4
    rng = np.random.default_rng(3)
    idx = _random_idx(rng, T, E, k)
    x = rng.integers(0, 0x7F00, size=(T, H), dtype=np.uint16)
    bounds, lays, so = _shard_layouts(idx, E, R)
    send, source_rows = _send_buffer(x, bounds, lays, k)
    rl = oracle.recv_layout(so, R)
    recv = oracle.exchange(send, source_rows, so, R)
    grouped = oracle.regroup(recv, so, R)
    whole = oracle.dispatch_layout(idx, E, R)
    np.testing.assert_array_equal(rl.group_offsets, whole.expert_offsets)
    np.testing.assert_array_equal(rl.recv_offsets[:, 0], whole.rank_offsets[:-1])
    np.testing.assert_array_equal(grouped, oracle.dispatch_pack(x, whole.pos, 0))
    if E == R or R == 1:   # one expert per rank, or one source: nothing moves
        np.testing.assert_array_equal(grouped, recv)


def test_regroup_brute_force_token_order():
    """Each expert's grouped rows are exactly the tokens that chose it, in
    ascending token id (numpy stable argsort as the reference)."""
    T, H, E, k, R = 300, 16, 16, 3, 4
    idx = _random_idx(np.random.default_rng(5), T, E, k)
    x = _tagged_rows(T, H)
    bounds, lays, so = _shard_layouts(idx, E, R)
    send, source_rows = _send_buffer(x, bounds, lays, k)
    rl = oracle.recv_layout(so, R)
    grouped = oracle.regroup(oracle.exchange(send, source_rows, so, R), so, R)
    g16 = grouped.view(np.uint16)
    tok = g16[:, 0].astype(np.int64) | (g16[:, 1].astype(np.int64) << 16)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(tok[:T * k], order // k)
    for e in range(E):
        seg = tok[rl.group_offsets[e]:rl.group_offsets[e + 1]]
        np.testing.assert_array_equal(seg, np.nonzero((idx == e).any(axis=1))[0])
    # segment starts: source s's rows of expert e come after those of sources < s
    for e in range(E):
        for s, (t0, t1) in enumerate(bounds):
            a = rl.group_seg[e, s]
            n = int(lays[s].expert_offsets[e + 1] - lays[s].expert_offsets[e])
            assert ((tok[a:a + n] >= t0) & (tok[a:a + n] < t1)).all()


def test_row_maps_are_inverse_permutations_and_drive_regroup():
    """group_pos is a bijection of [0, N) with inverse group_src, -1 past N;
    fancy indexing through the maps reproduces regroup in both directions."""
    T, H, E, k, R = 300, 16, 32, 4, 8
    idx = _random_idx(np.random.default_rng(8), T, E, k)
    x = _tagged_rows(T, H)
    bounds, lays, so = _shard_layouts(idx, E, R, cap=30)
    N = sum(l.n_rows for l in lays)
    rl = oracle.recv_layout(so, R, max_rows=N + 17)
    gp, gsrc = rl.group_pos, rl.group_src
    assert (gp[N:] == -1).all() and (gsrc[N:] == -1).all()
    np.testing.assert_array_equal(np.sort(gp[:N]), np.arange(N))
    np.testing.assert_array_equal(gsrc[gp[:N]], np.arange(N))
    send, source_rows = _send_buffer(x, bounds, lays, k)
    recv = oracle.exchange(send, source_rows, so, R)
    grouped = oracle.regroup(recv, so, R)
    np.testing.assert_array_equal(grouped[:N], recv[gsrc[:N]])
    np.testing.assert_array_equal(recv[:N], grouped[gp[:N]])


def test_round_trips_are_identity():
    T, H, E, k, R = 257, 32, 16, 2, 4       # ragged last source
    rng = np.random.default_rng(6)
    idx = _random_idx(rng, T, E, k)
    x = rng.integers(0, 0x7F00, size=(T, H), dtype=np.uint16)
    bounds, lays, so = _shard_layouts(idx, E, R)
    send, source_rows = _send_buffer(x, bounds, lays, k, quant=1)
    recv = oracle.exchange(send, source_rows, so, R)
    grouped = oracle.regroup(recv, so, R)
    back = oracle.regroup(np.zeros_like(recv), so, R, grouped=grouped, reverse=True)
    np.testing.assert_array_equal(back, recv)
    ret = oracle.exchange(np.zeros_like(send), source_rows, so, R, recv=back, reverse=True)
    for s, (t0, t1) in enumerate(bounds):
        n = lays[s].n_rows
        np.testing.assert_array_equal(ret[s * source_rows:s * source_rows + n],
                                      send[s * source_rows:s * source_rows + n])


def test_all_rows_to_one_rank_and_empty_sources():
    """Every token picks experts of rank 0; sources beyond T tokens are empty."""
    T, H, E, k, R = 5, 16, 16, 2, 8        # sources 5..7 hold no token
    idx = np.tile(np.array([[1, 0]], dtype=np.int32), (T, 1))
    x = _tagged_rows(T, H)
    bounds, lays, so = _shard_layouts(idx, E, R)
    assert bounds[-1][0] == bounds[-1][1]
    rl = oracle.recv_layout(so, R)
    assert rl.recv_offsets[0, R] == T * k and (rl.recv_offsets[1:] == T * k).all()
    send, source_rows = _send_buffer(x, bounds, lays, k)
    grouped = oracle.regroup(oracle.exchange(send, source_rows, so, R), so, R)
    g16 = grouped.view(np.uint16)
    np.testing.assert_array_equal(g16[:T, 0], np.arange(T))        # expert 0 first
    np.testing.assert_array_equal(g16[T:2 * T, 0], np.arange(T))   # then expert 1


@pytest.mark.parametrize("quant,cf", [(0, None), (1, None), (0, 1.25), (1, 1.25)])
def test_ep_layer_equals_chunked_layer(quant, cf):
    """The R-rank round trip through exchange and regroup returns the same
    bytes as the chunked layer with one chunk per source shard, capacity
    (per shard) included; a bias on expert 0 forces drops."""
    T, H, E, k, R = 512, 64, 16, 4, 4
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if cf:
        logits[:, 0] += 3.0
    x = oracle.floats_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    ep = oracle.run_ep_layer(logits, x, E, k, R, quant=quant, capacity_factor=cf)
    ref = oracle.run_layer(logits, x, E, k, R, chunks=R, quant=quant, capacity_factor=cf,
                           standin=True)
    if cf:
        assert sum(int((l.pos < 0).sum()) for l in ep.layouts) > 0
    np.testing.assert_array_equal(ep.out, ref.out)


def test_recv_layout_rejects_bad_shapes():
    so = np.zeros((3, 9), dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.recv_layout(so, 3)           # E=8 not divisible by R=3
    so = np.zeros((2, 9), dtype=np.int32)
    so[0, 3] = -1                           # decreasing offsets: negative count
    with pytest.raises(ValueError):
        oracle.recv_layout(so, 2)
    so = np.zeros((2, 9), dtype=np.int32)
    so[:, 1:] = 3                           # 6 rows do not fit 5 map entries
    with pytest.raises(ValueError):
        oracle.recv_layout(so, 2, max_rows=5)
