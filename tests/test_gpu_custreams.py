"""The dispatch/combine path on CU-masked streams: the output is bit for bit
that of the default stream, alone and while a GEMM runs concurrently on the
complementary CUs (whose result is unchanged too)."""
import numpy as np
import pytest
import torch

from combine_fp32_router_amd import custreams as CS
from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
def test_masked_streams_give_identical_results(quant):
    wl = I.WORKLOADS["mid"]
    x, logits = dev(I.make_hidden(wl)), dev(I.make_logits(wl))
    path = D.DispatchCombine(wl.T, wl.H, wl.E, wl.k, wl.R, chunks=2, ring=2, standin=True)
    ref = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    path.run(logits, x, ref, quant=quant)
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(2048, 2048, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(2048, 2048, device="cuda", generator=g).to(torch.bfloat16)
    c_ref = torch.matmul(a, b)
    torch.cuda.synchronize()
    for q in (1, 2, 3):
        data, comp = CS.split_streams(q)
        try:
            out = torch.empty_like(ref)
            with torch.cuda.stream(data.stream):
                path.run(logits, x, out, quant=quant)
            data.stream.synchronize()
            assert torch.equal(out, ref), f"masked {q}/4 alone"
            out2 = torch.empty_like(ref)
            c = torch.empty_like(c_ref)
            for _ in range(3):  # concurrently with a GEMM on the other CUs
                with torch.cuda.stream(data.stream):
                    path.run(logits, x, out2, quant=quant)
                with torch.cuda.stream(comp.stream):
                    torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
            assert torch.equal(out2, ref), f"masked {q}/4 with a concurrent GEMM"
            np.testing.assert_allclose(c.float().cpu().numpy(), c_ref.float().cpu().numpy(),
                                       rtol=1e-2, atol=1e-2)
        finally:
            data.close()
            comp.close()
