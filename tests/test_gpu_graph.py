"""The layer captured as a HIP graph (driver.capture) and replayed: every
replay equals an eager one-stream run on the same inputs bit for bit,
including replays after the inputs were rewritten in place and with eager
work through the same driver between replays (a replay must not depend on
state left by the capture).  Covers merged combine+pack launches, int8, a
capacity factor (per-chunk capacity table cached before capture), one
chunk, and the two-stream driver, whose event fork and joins become graph
edges."""
import numpy as np
import pytest
import torch

from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, E, k, R, chunks, quant, capacity factor, streams
    ("merged_bf16", 4096, 2048, 64, 8, 8, 4, 0, None, 1),
    ("merged_int8_cap", 4096, 2048, 64, 8, 8, 4, 1, 1.25, 1),
    ("merged_int4", 3001, 1024, 32, 6, 4, 3, 2, None, 1),
    ("one_chunk_fp8", 777, 512, 16, 2, 2, 1, 3, None, 1),
    ("two_streams_int8_cap", 8192, 1024, 128, 8, 16, 8, 1, 1.25, 2),
    ("two_streams_two_chunks", 1000, 512, 32, 4, 4, 2, 0, None, 2),
]


@pytest.mark.parametrize("name,T,H,E,k,R,chunks,quant,cf,streams", CASES,
                         ids=[c[0] for c in CASES])
def test_graph_replay_equals_eager(name, T, H, E, k, R, chunks, quant, cf, streams):
    wl = I.Workload(name, T=T, H=H, E=E, k=k, R=R, seed=9)
    x1, lg1 = dev(I.make_hidden(wl)), dev(I.make_logits(wl))
    wl2 = wl.with_(seed=10)
    x2, lg2 = dev(I.make_hidden(wl2)), dev(I.make_logits(wl2))
    eager = D.DispatchCombine(T, H, E, k, R, chunks=chunks)  # one stream: the reference
    ref = []
    for x, lg in ((x1, lg1), (x2, lg2)):
        o = torch.empty((T, H), dtype=torch.int16, device="cuda")
        eager.run(lg, x, o, quant=quant, capacity_factor=cf)
        torch.cuda.synchronize()
        ref.append(host(o))
    assert not np.array_equal(ref[0], ref[1])

    path = D.DispatchCombine(T, H, E, k, R, chunks=chunks, streams=streams)
    x_in, lg_in = x1.clone(), lg1.clone()
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    graph = D.capture(lambda: path.run(lg_in, x_in, out, quant=quant, capacity_factor=cf))
    for want, (x, lg) in [(0, (x1, lg1)), (1, (x2, lg2)), (0, (x1, lg1)), (0, (x1, lg1))]:
        x_in.copy_(x)
        lg_in.copy_(lg)
        out.fill_(0x5A5A)
        # eager work between replays, through the same driver: it rewrites
        # the staging and layout buffers the graph's launches use
        path.run(lg2 if want == 0 else lg1, x2 if want == 0 else x1, torch.empty_like(out),
                 quant=quant, capacity_factor=cf)
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), ref[want])
