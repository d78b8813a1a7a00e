"""The seeded synthetic workloads: determinism, shapes and structure."""
import numpy as np

from combine_fp32_router_amd import inputs


def test_deterministic_and_independent_streams():
    wl = inputs.WORKLOADS["tiny"]
    a, b = inputs.make_hidden(wl), inputs.make_hidden(wl)
    np.testing.assert_array_equal(a, b)
    # block size does not change the values
    np.testing.assert_array_equal(a, inputs.make_hidden(wl, rows_per_block=7))
    l0, l1 = inputs.make_logits(wl, 0), inputs.make_logits(wl, 1)
    assert l0.dtype == np.float32 and l0.shape == (wl.T, wl.E)
    assert not np.array_equal(l0, l1)
    assert not np.array_equal(inputs.make_hidden(wl.with_(seed=1)), a)


def test_distributions():
    wl = inputs.WORKLOADS["mid"]
    x = inputs.bf16_bits_to_f32(inputs.make_hidden(wl)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    l = inputs.make_logits(wl).astype(np.float64)
    assert abs(l.mean()) < 0.01 and abs(l.std() - 1) < 0.01


def test_dsv3_outliers_and_zipf_skew():
    wl = inputs.WORKLOADS["dsv3"].with_(H=64)
    rows = inputs.outlier_rows(wl)
    assert rows.size == round(0.01 * wl.T) == 164 and np.unique(rows).size == rows.size
    x = inputs.bf16_bits_to_f32(inputs.make_hidden(wl)).astype(np.float64)
    norms = np.sqrt((x * x).mean(1))
    assert np.all(norms[rows] > 20) and np.median(norms) < 2
    b = inputs.zipf_bias(wl.E, 1.1)
    assert b[0] == 0 and np.all(np.diff(b) < 0)
    l = inputs.make_logits(wl)
    top1 = np.argmax(l, axis=1)
    share = np.bincount(top1, minlength=wl.E) / wl.T
    assert share[0] == share.max() and share[0] > 0.2
