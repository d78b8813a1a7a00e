"""Host-side checks of the benchmark's contract (no GPU needed): more than
one GPU is refused with a message and a non-zero status before anything
touches a device, and the algorithmic byte counts follow the stated formula
(the 2*T*k*H*b exchange volume of the communication-wall explainer, plus the
token reads/writes and index traffic)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_formula():
    T, H, E, k = 16384, 7168, 256, 8
    b = bench.algorithmic_bytes(T, H, E, k, T * k, 0)
    assert b["pack"] + b["combine"] - 2 * T * H * 2 - T * k * 12 == 2 * T * k * H * 2  # 2TkHb
    assert b["route"] == T * E * 4 + T * k * 8
    assert b["total"] == 4248829952                      # 4.249 GB per step at this shape
    # quantised rows: codes plus the 4-byte scale kept beside them
    assert bench.payload_bytes(H, 1) == H + 4 and bench.payload_bytes(H, 2) == H // 2 + 4
    assert bench.payload_bytes(H, 3) == H + 4 and bench.payload_bytes(H, 0) == 2 * H
    i8 = bench.algorithmic_bytes(T, H, E, k, T * k, 1)
    assert abs((i8["pack"] - T * H * 2 - T * k * 4) / (T * k * 2 * H) - 0.5003) < 1e-4


def _oracle_snapshot(wl, x, logits, quant, chunks):
    """A snapshot of the shape bench.snapshot() copies from the GPU, filled
    from the oracle itself (rows and scales split as the library keeps them)."""
    import oracle
    idx, w = oracle.route_topk(logits, wl.k)
    c = chunks - 1
    t0, t1 = bench.chunk_bounds(wl.T, chunks)[c]
    lay = oracle.dispatch_layout(idx[t0:t1], wl.E, wl.R)
    rec = oracle.dispatch_pack(x[t0:t1], lay.pos, quant, n_rows=lay.n_rows)
    rb = (2 * wl.H, wl.H, wl.H // 2, wl.H)[quant]
    return {"quant": quant, "chunks": chunks, "c": c, "t0": t0, "t1": t1, "idx": idx, "w": w,
            "expert_counts": lay.expert_counts, "expert_offsets": lay.expert_offsets,
            "rank_counts": lay.rank_counts, "rank_offsets": lay.rank_offsets,
            "pos": lay.pos.ravel(), "row_src": lay.row_src,
            "send": np.ascontiguousarray(rec[:, :rb]),
            "scales": (np.ascontiguousarray(rec[:, rb:rb + 4]).view(np.float32).ravel()
                       if quant else None),
            "out": oracle.combine(rec, quant, lay.pos, w[t0:t1], wl.H)}


def test_parity_record_counts_and_bars():
    """bench.parity_check on the oracle's own results passes with zero
    mismatches; a code off by one is counted and allowed, by two it fails;
    a changed expert id or output element fails."""
    import oracle
    from combine_fp32_router_amd import inputs as I
    wl = I.Workload("p", T=96, H=64, E=8, k=2, R=2)
    x, logits = I.make_hidden(wl), I.make_logits(wl)
    for quant in (0, 1, 2, 3):
        snap = _oracle_snapshot(wl, x, logits, quant, 2)
        res = bench.parity_check(oracle, wl, snap, x, logits)
        assert res["pass"] and res["ids_mismatches"] == 0 and res["layout_mismatches"] == 0
        assert res.get("code_mismatches", 0) == 0 and res.get("bf16_element_mismatches", 0) == 0
    snap = _oracle_snapshot(wl, x, logits, 1, 2)
    codes = snap["send"].view(np.int8)
    j = int(np.argmin(np.abs(codes[0].astype(int))))  # a small code: +1 / +2 stay in range
    codes[0, j] += 1
    res = bench.parity_check(oracle, wl, snap, x, logits)
    assert res["code_mismatches"] == 1 and res["max_code_diff"] == 1 and res["pass"]
    codes[0, j] += 1
    assert not bench.parity_check(oracle, wl, snap, x, logits)["pass"]
    snap = _oracle_snapshot(wl, x, logits, 0, 2)
    snap["idx"] = snap["idx"].copy()
    snap["idx"][3, 0] = (snap["idx"][3, 0] + 1) % wl.E
    res = bench.parity_check(oracle, wl, snap, x, logits)
    assert res["ids_mismatches"] == 1 and not res["pass"]
    snap = _oracle_snapshot(wl, x, logits, 0, 2)
    snap["out"] = snap["out"].copy()
    snap["out"][0, 0] ^= 0x0100  # one element off by far more than the bar
    res = bench.parity_check(oracle, wl, snap, x, logits)
    assert res["out_violations"] == 1 and not res["pass"]
    snap["out"][0, 0] = 0x7FC0    # a NaN fails too
    res = bench.parity_check(oracle, wl, snap, x, logits)
    assert res["out_nonfinite"] == 1 and res["out_violations"] == 1 and not res["pass"]


def test_inputs_alternate_two_equal_copies():
    """Every timed leg reads input copy s % 2 at step s: consecutive steps get
    different buffers holding the same values (so no step finds the previous
    step's inputs in the last-level cache, and every step computes the same
    result)."""
    import torch
    x = torch.arange(12, dtype=torch.int16).view(3, 4)
    lg = [torch.randn(3, 8), torch.randn(3, 8)]
    inp = bench.Inputs(x, lg)
    (x0, l0), (x1, l1), (x2, l2) = inp(0), inp(1), inp(2)
    assert x0 is x and x2 is x0 and l2[0] is l0[0]
    assert x1.data_ptr() != x0.data_ptr() and torch.equal(x1, x0)
    for a, b in zip(l0, l1):
        assert a.data_ptr() != b.data_ptr() and torch.equal(a, b)


def test_weight_error_handles_underflowed_weights():
    """The parity record's weight error: relative where the reference weight
    is nonzero; a reference weight of exactly 0 (underflow) must be matched
    by 0, anything else (or a NaN) is an infinite error."""
    r = np.array([0.5, 0.0, 0.25, 1e-45], np.float32)
    assert bench.weights_max_rel_err(r, r) == 0.0
    g = r.copy()
    g[2] = np.nextafter(np.float32(0.25), np.float32(1))
    assert 0 < bench.weights_max_rel_err(g, r) < 1e-6
    g = r.copy()
    g[1] = np.float32(1e-30)
    assert bench.weights_max_rel_err(g, r) == np.inf
    g = r.copy()
    g[0] = np.nan
    assert bench.weights_max_rel_err(g, r) == np.inf
