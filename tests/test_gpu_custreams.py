"""The dispatch/combine path on CU-masked streams (communication confined to
a slice of the CUs so a concurrent computation keeps the rest, the rate
limiting of the ThunderEP write-up, s2.2), checked against the oracle's
layer: expert ids bit-exact and outputs within 1e-3 + 1e-2*|ref|, alone and
while a GEMM runs on the complementary CUs (whose result is checked too);
the masked output also equals the default stream's bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from combine_fp32_router_amd import custreams as CS
from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I
from gpu_util import assert_out_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
def test_masked_streams_match_the_oracle(quant):
    wl = I.WORKLOADS["mid"]
    x_h, logits_h = I.make_hidden(wl), I.make_logits(wl)
    print(f"custreams: mid T={wl.T} H={wl.H} quant={quant}", flush=True)
    ref = oracle.run_layer(logits_h, x_h, wl.E, wl.k, wl.R, chunks=2, quant=quant, standin=True,
                           keep_buffers=False, workers=8)
    x, logits = dev(x_h), dev(logits_h)
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=2, ring=2, standin=True)
    plain = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    path.run(logits, x, plain, quant=quant)
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(2048, 2048, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(2048, 2048, device="cuda", generator=g).to(torch.bfloat16)
    c_ref = torch.matmul(a.float(), b.float())
    torch.cuda.synchronize()
    assert_out_close(host(plain), ref.out, "default stream")
    for q in (1, 2, 3):
        data, comp = CS.split_streams(q)
        try:
            out = torch.empty_like(plain)
            with torch.cuda.stream(data.stream):
                path.run(logits, x, out, quant=quant)
            data.stream.synchronize()
            np.testing.assert_array_equal(host(path.idx), ref.idx)
            assert_out_close(host(out), ref.out, f"masked {q}/4 alone")
            assert torch.equal(out, plain), f"masked {q}/4 alone vs the default stream"
            out2 = torch.empty_like(plain)
            c = torch.empty((2048, 2048), dtype=torch.bfloat16, device="cuda")
            for _ in range(3):  # concurrently with a GEMM on the other CUs
                with torch.cuda.stream(data.stream):
                    path.run(logits, x, out2, quant=quant)
                with torch.cuda.stream(comp.stream):
                    torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(path.idx), ref.idx)
            assert_out_close(host(out2), ref.out, f"masked {q}/4 beside a GEMM")
            assert torch.equal(out2, plain), f"masked {q}/4 beside a GEMM vs the default stream"
            np.testing.assert_allclose(c.float().cpu().numpy(), c_ref.cpu().numpy(),
                                       rtol=2e-2, atol=2e-1)
        finally:
            data.close()
            comp.close()
