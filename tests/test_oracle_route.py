"""Pins for the oracle's routing step (O1): top-k selection and gate weights.

Each test checks the oracle against something other than itself: the
router example printed on the communication-wall page, numpy's argmax /
stable argsort, scipy's softmax, closed forms and brute force.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(int, ln.split())) for ln in f if ln.strip() and not ln.startswith("#")]


def test_router_example_from_page():
    """Communication-wall page, router example: token1 -> E3, E17; token2 ->
    E8, E22; token3 -> E3, E11 (k=2).  Logits put the named experts on top in
    the printed order; the rest stay below."""
    rows = _rows("commwall_router_example.txt")
    E, k = 32, 2
    rng = np.random.default_rng(1)
    logits = (rng.standard_normal((len(rows), E)) * 0.1 - 3.0).astype(np.float32)
    for i, (_, a, b) in enumerate(rows):
        logits[i, a] = 2.0
        logits[i, b] = 1.0
    idx, w = oracle.route_topk(logits, k)
    assert idx.tolist() == [[a, b] for _, a, b in rows]
    # w0 = 1 / (1 + e^(l1 - l0)) = 1 / (1 + e^-1) for both logit pairs
    assert np.allclose(w[:, 0], 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-7)
    # the bucket of expert 3 holds token 1 then token 3
    lay = oracle.dispatch_layout(idx, E, R=4)
    r3 = lay.row_src[lay.expert_offsets[3]:lay.expert_offsets[4]]
    assert (r3 // k).tolist() == [0, 2]


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 8), (256, 8), (37, 5)])
def test_matches_numpy_stable_argsort(E, k):
    """Selection = first k of a stable descending sort (ties -> lower id).
    Logits are rounded to 1/4 so that ties are frequent."""
    rng = np.random.default_rng(E * 100 + k)
    logits = (np.round(rng.standard_normal((300, E)) * 4) / 4).astype(np.float32)
    idx, _ = oracle.route_topk(logits, k)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref)


def test_k1_is_numpy_argmax():
    rng = np.random.default_rng(7)
    logits = (np.round(rng.standard_normal((500, 16)) * 2) / 2).astype(np.float32)
    idx, w = oracle.route_topk(logits, 1)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(logits, axis=1))
    assert np.all(w == 1.0)  # a single selected expert gets weight exactly 1


def test_all_equal_logits():
    for E, k in [(8, 2), (64, 8), (5, 5)]:
        logits = np.full((3, E), 0.75, dtype=np.float32)
        idx, w = oracle.route_topk(logits, k)
        assert (idx == np.arange(k)).all()
        np.testing.assert_allclose(w, 1.0 / k, rtol=1e-7)


def test_signed_zero_is_a_tie():
    """-0.0 and +0.0 compare equal, so the lower id wins either way."""
    logits = np.array([[0.0, -0.0, -1.0], [-0.0, 0.0, -1.0]], dtype=np.float32)
    idx, _ = oracle.route_topk(logits, 1)
    assert idx[:, 0].tolist() == [0, 0]


def test_brute_force_small():
    """E <= 6: the selected set is the k-subset maximising the sorted value
    vector, ties broken towards lower ids; output order descending."""
    rng = np.random.default_rng(3)
    for E in (2, 3, 5, 6):
        for k in range(1, E + 1):
            logits = rng.integers(-2, 3, size=(40, E)).astype(np.float32)
            idx, _ = oracle.route_topk(logits, k)
            for t in range(logits.shape[0]):
                l = logits[t]
                best = None
                for sub in itertools.combinations(range(E), k):
                    key = sorted(((-l[e], e) for e in sub))
                    if best is None or key < best:
                        best = key
                assert idx[t].tolist() == [e for _, e in best]
                sel = set(idx[t].tolist())
                for e in range(E):
                    if e not in sel:
                        assert all(l[s] >= l[e] for s in sel)


def test_weights_sum_and_full_softmax():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((200, 16)).astype(np.float32) * 3
    _, w = oracle.route_topk(logits, 4)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, rtol=0, atol=1e-6)
    # k = E: weights are the textbook full softmax, in descending order
    idx, w = oracle.route_topk(logits, 16)
    ref = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, idx, 1), rtol=1e-6)


def test_weights_are_renormalised_full_softmax():
    """Renormalising the full softmax over the top-k gives the same weights."""
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((100, 64)).astype(np.float32)
    idx, w = oracle.route_topk(logits, 8)
    p = softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6)


def test_k2_logistic_closed_form():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((100, 8)).astype(np.float32)
    idx, w = oracle.route_topk(logits, 2)
    d = np.take_along_axis(logits, idx, 1).astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(d[:, 1] - d[:, 0])), rtol=1e-6)
    np.testing.assert_allclose(w[:, 1], 1.0 / (1.0 + np.exp(d[:, 0] - d[:, 1])), rtol=1e-6)


def test_shift_invariance():
    """Adding a constant to a token's logits changes neither the experts nor
    the weights (integers: the shift is exact in fp32)."""
    rng = np.random.default_rng(9)
    logits = rng.integers(-20, 20, size=(100, 32)).astype(np.float32)
    i0, w0 = oracle.route_topk(logits, 8)
    i1, w1 = oracle.route_topk(logits + np.float32(1000.0), 8)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_allclose(w0, w1, rtol=1e-6)


def test_descending_order():
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((100, 64)).astype(np.float32)
    idx, w = oracle.route_topk(logits, 8)
    v = np.take_along_axis(logits, idx, 1)
    assert np.all(np.diff(v, axis=1) <= 0)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_rejects_non_finite():
    logits = np.zeros((2, 4), dtype=np.float32)
    logits[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.route_topk(logits, 2)
    logits[1, 2] = np.inf
    with pytest.raises(ValueError):
        oracle.route_topk(logits, 2)


def _fp32_round_exact(v):
    """The fp32 value nearest the Decimal v > 0 (ties to even), or None when
    v lies within 1e-13 (relative) of the midpoint between two fp32 values,
    where a double evaluation may round either way."""
    from decimal import Decimal
    f = np.float32(float(v))
    lo = f if Decimal(float(f)) <= v else np.nextafter(f, np.float32(0))
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (Decimal(float(lo)) + Decimal(float(hi))) / 2
    if abs(v - mid) <= v * Decimal("1e-13"):
        return None
    return lo if v < mid else hi


def test_weights_are_the_correctly_rounded_fp32_of_the_exact_value():
    """The last ulp of the fp32 gate weights: each weight is the exact
    renormalised softmax exp(l_j - l_max) / sum_i exp(l_i - l_max) over the
    selected logits, evaluated in 60-digit decimal arithmetic (independent
    of the oracle's double evaluation and its libm), rounded once to fp32.
    Values within 1e-13 of an fp32 rounding midpoint are counted, not
    compared (double evaluation is accurate to ~1e-15 there).  Includes
    tokens whose weights are fp32 subnormals."""
    from decimal import Decimal, localcontext
    rng = np.random.default_rng(21)
    logits = (rng.standard_normal((300, 64)) * 3).astype(np.float32)
    logits[:4, :8] = np.array([0, -30, -60, -87, -92, -96, -99, -101], np.float32)
    logits[:4, 8:] = -200
    idx, w = oracle.route_topk(logits, 8)
    assert np.all((w[:4, 7] > 0) & (w[:4, 7] < np.finfo(np.float32).tiny))  # subnormal weights
    compared = skipped = 0
    with localcontext() as ctx:
        ctx.prec = 60
        for t in range(logits.shape[0]):
            sel = [Decimal(float(logits[t, e])) for e in idx[t]]
            top = max(sel)
            ex = [(l - top).exp() for l in sel]
            tot = sum(ex)
            for j in range(8):
                want = _fp32_round_exact(ex[j] / tot)
                if want is None:
                    skipped += 1
                    continue
                compared += 1
                assert w[t, j] == want, (t, j, w[t, j], want)
    assert compared >= 2390 and skipped <= 10
