"""Pins of the oracle's 4-bit payload (ThunderEP write-up s5.2: 4-bit as the
next, more aggressive compression step).  Reading: the int8 rule with 4-bit
codes -- scale = max|x|/7, code = rne(x/scale) clamped to [-7, 7], two codes
per byte (element 2i in the low nibble, 4-bit two's complement), record =
H/2 code bytes + fp32 scale + 12 zero bytes."""
import numpy as np
import pytest

import oracle
from combine_fp32_router_amd import inputs


def _f32(bits):
    return inputs.bf16_bits_to_f32(bits)


def _bits(vals):
    a = np.asarray(vals, dtype=np.float32)
    assert np.array_equal(_f32((a.view(np.uint32) >> 16).astype(np.uint16)), a)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _codes(rec, H):
    """Unpack nibbles independently of the oracle: low nibble first."""
    b = rec[:H // 2].astype(np.int32)
    lo, hi = b & 0xF, b >> 4
    c = np.empty(H, dtype=np.int32)
    c[0::2], c[1::2] = lo, hi
    return np.where(c >= 8, c - 16, c)


def test_int4_volume_about_quarter():
    for H, ratio in [(7168, 0.2511), (4096, 0.2520), (512, 0.2656)]:
        assert oracle.record_bytes(H, 2) == H // 2 + 16
        assert abs(oracle.record_bytes(H, 2) / oracle.record_bytes(H, 0) - ratio) < 1e-4


def test_int4_hand_worked_ties_and_nibbles():
    """max|x| = 7 gives scale exactly 1.0 (codes = x rounded half to even);
    max|x| = 14 gives scale exactly 2.0.  The packed bytes are written out by
    hand: byte i = code(2i) & 0xF | (code(2i+1) & 0xF) << 4."""
    H = 16
    r1 = [2.5, 3.5, -2.5, 0.5, 1.5, 7.0, -7.0, 0.0, 1.0, -1.0, 6.5, 0.25, -0.75, 5.5, -5.5, 4.0]
    r2 = [5.0, 7.0, -14.0, 1.0, 3.0, 0.0, 2.0, -6.0, 10.0, 11.0, 13.0, 9.0, -3.0, 14.0, 0.5, -1.0]
    x = np.stack([_bits(r1), _bits(r2)])
    send = oracle.dispatch_pack(x, np.array([[0], [1]], dtype=np.int32), 2)
    assert send.shape == (2, H // 2 + 16)
    assert send[0, :8].tolist() == [0x42, 0x0E, 0x72, 0x09, 0xF1, 0x06, 0x6F, 0x4A]
    assert _codes(send[0], H).tolist() == [2, 4, -2, 0, 2, 7, -7, 0, 1, -1, 6, 0, -1, 6, -6, 4]
    assert _codes(send[1], H).tolist() == [2, 4, -7, 0, 2, 0, 1, -3, 5, 6, 6, 4, -2, 7, 0, 0]
    assert send[:, 8:12].copy().view(np.float32).ravel().tolist() == [1.0, 2.0]
    assert (send[:, 12:] == 0).all()


def test_int4_closed_form_bounds():
    """Largest |x| maps to +-7 with its sign; |q*scale - x| <= scale*(1/2 +
    2^-16); a zero row gives zero codes and scale 0; nibble 8 (-8) unused."""
    wl = inputs.Workload("t", T=300, H=256, E=8, k=2, R=2, outlier_frac=0.05)
    x = inputs.make_hidden(wl)
    x[7] = 0
    send = oracle.dispatch_pack(x, np.arange(wl.T, dtype=np.int32)[:, None], 2)
    H = wl.H
    codes = np.stack([_codes(r, H) for r in send]).astype(np.float64)
    scale = send[:, H // 2:H // 2 + 4].copy().view(np.float32).ravel().astype(np.float64)
    xf = _f32(x).astype(np.float64)
    amax = np.abs(xf).max(1)
    assert scale[7] == 0 and (codes[7] == 0).all()
    nz = amax > 0
    np.testing.assert_allclose(scale[nz], amax[nz] / 7, rtol=2 ** -23)
    am = np.argmax(np.abs(xf), axis=1)
    top = codes[np.arange(wl.T), am]
    assert np.all(np.abs(top[nz]) == 7)
    assert np.all(np.sign(top[nz]) == np.sign(xf[np.arange(wl.T), am][nz]))
    assert np.all(np.abs(codes * scale[:, None] - xf) <= scale[:, None] * (0.5 + 2 ** -16))
    assert codes.min() >= -7 and codes.max() <= 7


def test_int4_k1_roundtrip_within_half_step():
    """k = 1, no expert: out = bf16(q * scale), within half a quantisation
    step of x plus one bf16 rounding."""
    wl = inputs.Workload("t", T=200, H=128, E=16, k=1, R=4)
    x = inputs.make_hidden(wl)
    res = oracle.run_layer(inputs.make_logits(wl), x, wl.E, 1, wl.R, chunks=2, quant=2)
    xf = _f32(x).astype(np.float64)
    step = np.abs(xf).max(1, keepdims=True) / 7
    out = _f32(res.out).astype(np.float64)
    assert np.all(np.abs(out - xf) <= step * 0.5 * (1 + 2 ** -7) + np.abs(xf) * 2 ** -8 + 1e-30)


def test_standin_int4_return_path_closed_form():
    wl = inputs.WORKLOADS["tiny"].with_(H=256)
    x = inputs.make_hidden(wl)
    res = oracle.run_layer(inputs.make_logits(wl), x, wl.E, wl.k, wl.R, chunks=2, quant=2,
                           standin=True)
    xf = _f32(x).astype(np.float64)
    f = (res.w.astype(np.float64) * (1 + res.idx / 8.0)).sum(1)
    ref = xf * f[:, None]
    # two int4 round trips (dispatch, return), each <= half a step of the row max
    amax = np.abs(xf).max(1, keepdims=True) * (1 + wl.E / 8.0)
    assert np.all(np.abs(_f32(res.out) - ref) <= 2 * 0.5 * amax / 7 * 1.05 + 1e-2 * np.abs(ref))


def test_int4_roundtrip_token_matches_full_path():
    wl = inputs.Workload("t", T=64, H=96, E=8, k=3, R=2, outlier_frac=0.1)
    x = inputs.make_hidden(wl)
    res = oracle.run_layer(inputs.make_logits(wl), x, wl.E, wl.k, wl.R, chunks=1, quant=2)
    pos = res.layouts[0].pos
    for t in (0, 5, 63):
        np.testing.assert_array_equal(oracle.roundtrip_token(x[t], pos[t], res.w[t], 2), res.out[t])


def test_int4_rejects_odd_hidden():
    x = np.zeros((2, 15), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.dispatch_pack(x, np.array([[0], [1]], dtype=np.int32), 2)
