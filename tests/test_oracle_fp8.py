"""Pins of the oracle's fp8 payload (OCP E4M3; the NCCL EP article's s6.3
FP8 communication).  Reading: the int8 rule with an E4M3 code -- scale =
max|x|/448, code = E4M3(x/scale) round to nearest even, record = H codes +
fp32 scale + 12 zero bytes."""
import numpy as np

import oracle
from combine_fp32_router_amd import inputs


def _f32(bits):
    return inputs.bf16_bits_to_f32(bits)


def _bits(vals):
    a = np.asarray(vals, dtype=np.float32)
    assert np.array_equal(_f32((a.view(np.uint32) >> 16).astype(np.uint16)), a)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _e4m3_values():
    """Closed form of every code (independent of the oracle): sign, 4-bit
    exponent with bias 7, 3-bit mantissa; exponent 0 is subnormal."""
    c = np.arange(256)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    v = s * mag
    v[(e == 15) & (m == 7)] = np.nan
    return v


def test_decode_all_codes():
    ref = _e4m3_values()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_encode_hand_cases():
    cases = [(0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE),
             (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (0.5 * 2.0 ** -9, 0x00),
             (0.75 * 2.0 ** -9, 0x01), (1.0625, 0x38), (1.1875, 0x3A), (240.0, 0x77),
             (460.0, 0x7E), (-3.0, 0xC4)]
    for v, c in cases:  # pairs, not a dict: 0.0 and -0.0 are equal keys
        assert oracle.e4m3_encode(v) == c, (v, hex(oracle.e4m3_encode(v)), hex(c))


def test_encode_is_nearest_code_ties_to_even():
    """Brute force over the finite non-negative codes: the encoder picks the
    nearest value, and on an exact tie the code with the even mantissa."""
    vals = _e4m3_values()[:0x7F]                 # 0x00..0x7E, increasing
    rng = np.random.default_rng(0)
    mids = 0.5 * (vals[1:] + vals[:-1])
    xs = np.concatenate([rng.uniform(0, 460, 4000), rng.uniform(0, 1, 4000) * 2.0 ** -5,
                         mids, vals]).astype(np.float32)
    for x in xs.tolist():
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert oracle.e4m3_encode(x) == want, x
        assert oracle.e4m3_encode(-x) == (want | 0x80), x


def test_round_trip_every_finite_code():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c


def test_fp8_record_hand_worked():
    """max|x| = 448 makes the scale exactly 1: codes are E4M3(x)."""
    H = 16
    row = [448.0, -448.0, 1.0, 1.0625, 1.1875, 240.0, -3.0, 0.0, 2.0 ** -6, 2.0 ** -9,
           0.5, 100.0, -0.25, 7.0, 56.0, 3.5]
    send = oracle.dispatch_pack(_bits(row)[None, :], np.array([[0]], dtype=np.int32), 3)
    assert send.shape == (1, H + 16)
    assert send[0, :H].tolist() == [oracle.e4m3_encode(v) for v in row]
    assert send[0, :3].tolist() == [0x7E, 0xFE, 0x38]
    assert send[0, H:H + 4].copy().view(np.float32)[0] == 1.0
    assert (send[0, H + 4:] == 0).all()


def test_fp8_closed_form_bounds():
    """The largest |x| maps to +-448; every element is within half an E4M3
    step of x/scale (relative 2^-4 for normals, 2^-10 absolute below 2^-6);
    a zero row gives zero codes and scale 0."""
    wl = inputs.Workload("t", T=300, H=256, E=8, k=2, R=2, outlier_frac=0.05)
    x = inputs.make_hidden(wl)
    x[7] = 0
    send = oracle.dispatch_pack(x, np.arange(wl.T, dtype=np.int32)[:, None], 3)
    H = wl.H
    vals = _e4m3_values()
    q = vals[send[:, :H]]
    scale = send[:, H:H + 4].copy().view(np.float32).ravel().astype(np.float64)
    xf = _f32(x).astype(np.float64)
    amax = np.abs(xf).max(1)
    assert scale[7] == 0 and (send[7, :H] == 0).all()
    nz = amax > 0
    np.testing.assert_allclose(scale[nz], amax[nz] / 448, rtol=2 ** -23)
    am = np.argmax(np.abs(xf), axis=1)
    assert np.all(np.abs(q[np.arange(wl.T), am][nz]) == 448)
    y = xf[nz] / scale[nz, None]
    err = np.abs(q[nz] - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))


def test_fp8_roundtrip_token_matches_full_path_and_standin():
    wl = inputs.Workload("t", T=64, H=96, E=8, k=3, R=2, outlier_frac=0.1)
    x = inputs.make_hidden(wl)
    res = oracle.run_layer(inputs.make_logits(wl), x, wl.E, wl.k, wl.R, chunks=1, quant=3)
    pos = res.layouts[0].pos
    for t in (0, 5, 63):
        np.testing.assert_array_equal(oracle.roundtrip_token(x[t], pos[t], res.w[t], 3), res.out[t])
    # stand-in on the fp8 return path: within two fp8 round trips of the closed form
    res = oracle.run_layer(inputs.make_logits(wl), x, wl.E, wl.k, wl.R, chunks=1, quant=3,
                           standin=True)
    xf = _f32(x).astype(np.float64)
    ref = xf * (res.w.astype(np.float64) * (1 + res.idx / 8.0)).sum(1)[:, None]
    amax = np.abs(xf).max(1, keepdims=True) * (1 + wl.E / 8.0)
    assert np.all(np.abs(_f32(res.out) - ref) <= 2 * 2.0 ** -4 * np.abs(ref) * 1.1
                  + 2 * 2.0 ** -10 * amax / 448 + 1e-2 * np.abs(ref) + 1e-6)


def test_fp8_volume_as_int8():
    for H in (7168, 512):
        assert oracle.record_bytes(H, 3) == oracle.record_bytes(H, 1) == H + 16
