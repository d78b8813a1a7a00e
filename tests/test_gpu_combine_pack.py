"""GPU parity of moe_combine_pack (combine of one chunk and pack of another
in one launch): its outputs equal the two separate calls bit for bit, with
either store policy for the send rows (MOE_PACK_STREAM or not), and
the oracle's combine and pack to the usual bars (outputs 1e-3 abs + 1e-2
rel; bf16 records bitwise, quantised codes +-1).  Cases cover ragged and
empty halves, dropped slots, and hidden sizes whose row tiling takes 2, 4
and 8 vectors per thread (int4 then packs with half the combine's)."""
import numpy as np
import pytest
import torch

import oracle
from combine_fp32_router_amd import binding as B
from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I
from gpu_util import (assert_out_close, compare_records, dev, dev_rows, host,
                      join_records, row_bytes)

pytestmark = pytest.mark.gpu

CASES = [
    # name, Tc (combine tokens), Tp (pack tokens), H, E, k, capacity (0: none)
    ("ragged", 300, 257, 7168, 64, 8, 0),
    ("combine_only", 200, 0, 2048, 16, 4, 0),
    ("pack_only", 0, 199, 2048, 16, 4, 0),
    ("one_each", 1, 1, 512, 8, 2, 0),
    ("drops", 257, 300, 1024, 32, 6, 20),
    ("H32768", 40, 33, 32768, 16, 4, 0),
    ("H65536", 9, 12, 65536, 8, 2, 0),
]


def half(name, T, H, E, k, cap, quant, seed):
    """Inputs of one half: hidden rows, routing, layout and, for the combine
    half, the records the oracle's pack writes for them."""
    wl = I.Workload(name, T=T, H=H, E=E, k=k, R=1, seed=seed)
    x = I.make_hidden(wl)
    idx, w = oracle.route_topk(I.make_logits(wl), k)
    lay = oracle.dispatch_layout(idx, E, 1, cap)
    recs = oracle.dispatch_pack(x, lay.pos, quant)
    return x, w, lay, recs


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
@pytest.mark.parametrize("name,Tc,Tp,H,E,k,cap", CASES, ids=[c[0] for c in CASES])
def test_combine_pack_parity(name, Tc, Tp, H, E, k, cap, quant):
    rb = row_bytes(H, quant)
    if Tc:
        _, wc, layc, recv = half(name + "_c", Tc, H, E, k, cap, quant, 11)
    if Tp:
        xp, _, layp, _ = half(name + "_p", Tp, H, E, k, cap, quant, 12)
    rows_p = max(Tp * k, 1)
    recv_d, recv_s = dev_rows(recv, H, quant) if Tc else (None, None)
    pos_c = dev(layc.pos) if Tc else None
    w_c = dev(wc) if Tc else None
    x_p = dev(xp) if Tp else None
    pos_p = dev(layp.pos) if Tp else None
    outs, sends, scales = [], [], []
    # merged and separate launches, each with the default and the streaming
    # store policy for the send rows (MOE_PACK_STREAM): all four write the same
    for fused, flags in ((True, 0), (False, 0), (True, B.MOE_PACK_STREAM),
                         (False, B.MOE_PACK_STREAM)):
        out = torch.full((max(Tc, 1), H), 0x7BCD, dtype=torch.int16, device="cuda")
        send = torch.full((rows_p, rb), 0xAB, dtype=torch.uint8, device="cuda")
        send_s = torch.full((rows_p,), -3.0, dtype=torch.float32, device="cuda") if quant else None
        if fused:
            B.moe_combine_pack(recv_d, recv_s, pos_c, w_c, Tc, out, x_p, pos_p, Tp, send, send_s,
                               H, k, quant | flags)
        else:
            if Tc:
                B.moe_combine(recv_d, recv_s, quant, pos_c, w_c, Tc, H, k, out)
            if Tp:
                B.moe_dispatch_pack(x_p, Tp, H, k, pos_p, quant | flags, send, send_s)
        torch.cuda.synchronize()
        outs.append(host(out))
        sends.append(host(send))
        scales.append(host(send_s) if quant else np.zeros(rows_p, np.float32))
    for i in (1, 2, 3):
        np.testing.assert_array_equal(outs[0], outs[i])
        np.testing.assert_array_equal(sends[0], sends[i])
        np.testing.assert_array_equal(scales[0].view(np.int32), scales[i].view(np.int32))
    if Tc:
        assert_out_close(outs[0], oracle.combine(recv, quant, layc.pos, wc, H), f"{name} combine")
    else:
        assert (outs[0] == 0x7BCD).all(), "combine half wrote with Tc == 0"
    if Tp:
        N = layp.n_rows
        ref = oracle.dispatch_pack(xp, layp.pos, quant, n_rows=N)
        compare_records(join_records(sends[0][:N], scales[0][:N], H, quant), ref, H, quant,
                        f"{name} pack")
        assert (sends[0][N:] == 0xAB).all(), "pack wrote rows no slot points to"
        if quant:
            assert (scales[0][N:] == -3.0).all(), "pack wrote scales no slot points to"
    else:
        assert (sends[0] == 0xAB).all(), "pack half wrote with Tp == 0"
        assert (scales[0] == (-3.0 if quant else 0.0)).all(), "pack half wrote with Tp == 0"


def test_combine_pack_rejects_send_equal_recv():
    H, k = 512, 2
    buf = torch.zeros((8, 2 * H), dtype=torch.uint8, device="cuda")
    other = torch.zeros((8, 2 * H), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(8, dtype=torch.float32, device="cuda")
    pos = torch.zeros(4 * k, dtype=torch.int32, device="cuda")
    w = torch.zeros(4 * k, dtype=torch.float32, device="cuda")
    out = torch.zeros((4, H), dtype=torch.int16, device="cuda")
    x = torch.zeros((4, H), dtype=torch.int16, device="cuda")
    with pytest.raises(B.MoeError, match="ALIAS"):
        B.moe_combine_pack(buf, None, pos, w, 4, out, x, pos, 4, buf, None, H, k, 0)
    with pytest.raises(B.MoeError, match="ALIAS"):  # one scale array for both halves
        B.moe_combine_pack(buf, sc, pos, w, 4, out, x, pos, 4, other, sc, H, k, 1)


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
@pytest.mark.parametrize("standin", [False, True], ids=["identity", "standin"])
def test_driver_merged_equals_separate(quant, standin):
    """The whole layer with merged launches (C+1 big launches) equals the
    layer with separate pack and combine launches, bit for bit, for a
    ragged chunking and both staging-ring sizes that allow merging."""
    wl = I.Workload("merge", T=1001, H=1024, E=32, k=4, R=4, seed=5)
    x, logits = dev(I.make_hidden(wl)), dev(I.make_logits(wl))
    res = []
    for merge, ring, stream_stores in ((False, 2, False), (True, 2, False), (True, 3, False),
                                       (False, 2, True), (True, 2, True)):
        path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=5, ring=ring,
                                 standin=standin, merge=merge, stream_stores=stream_stores)
        out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
        timer = D.KernelTimer()
        path.run(logits, x, out, quant=quant, timer=timer)
        torch.cuda.synchronize()
        launches = {n: len(v) for n, v in timer.spans.items()}
        assert launches.get("combine_pack", 0) == (4 if merge else 0), launches
        res.append(host(out))
    for r in res[1:]:
        np.testing.assert_array_equal(res[0], r)


def test_driver_ring1_does_not_merge():
    """One staging buffer: the pack of chunk c+1 would overwrite the rows the
    combine of chunk c reads, so the driver keeps the launches apart."""
    wl = I.Workload("ring1", T=300, H=512, E=8, k=2, R=2, seed=6)
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=3, ring=1)
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    timer = D.KernelTimer()
    path.run(dev(I.make_logits(wl)), dev(I.make_hidden(wl)), out, quant=0, timer=timer)
    torch.cuda.synchronize()
    assert "combine_pack" not in timer.spans
    ref = oracle.run_layer(I.make_logits(wl), I.make_hidden(wl), wl.E, wl.k, wl.R, chunks=3,
                           quant=0)
    assert_out_close(host(out), ref.out, "ring1")
