"""The benchmark's HBM-only leg runs the ordinary pipeline's launches with
the exchange as a one-step delay line (combine of chunk c reads the rows
packed for chunk c a step earlier) and alternates two copies of the inputs
between steps.  Its output must equal the ordinary pipeline's bit for bit,
with either store policy for the send rows, so the figure it reports is for
the same computation."""
import argparse
import os
import sys

import numpy as np
import pytest
import torch

from combine_fp32_router_amd import driver as D
from combine_fp32_router_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["bf16", "int8", "int4", "fp8"])
@pytest.mark.parametrize("stream_stores", [True, False], ids=["streaming", "device"])
def test_delay_line_equals_pipeline(quant, stream_stores):
    wl = I.Workload("dl", T=3000, H=1024, E=32, k=4, R=4, seed=9, zipf_s=1.1)
    x = torch.from_numpy(I.make_hidden(wl).view(np.int16)).cuda()
    lg = torch.from_numpy(I.make_logits(wl)).cuda()
    args = argparse.Namespace(ring=2, unfused=False, no_merge=False, graph=False)
    for chunks in (1, 3, 4):
        print(f"delay line q={quant} stream={stream_stores} chunks={chunks}", flush=True)
        res = bench.measure_delayed(args, wl, quant, chunks, bench.Inputs(x, [lg]), torch, D,
                                    steps=3, warmup=2, stream_stores=stream_stores)
        assert res["output_equals_pipeline"], res
        assert res["algorithmic_bytes_per_step"] > 0 and res["ms_per_step"] > 0
