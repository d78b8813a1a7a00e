"""The test-support library's stream probe: the copy reproduces its source
exactly, including a short last tile, and writes nothing past it; the read
sweeps count the all-ones 16-byte vectors of their source, nothing else,
including those in a short last tile."""
import numpy as np
import pytest
import torch

from combine_fp32_router_amd import harness as HN

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 * 3 + 16, (1 << 22) + 48])
def test_copy_exact_with_ragged_tail(nbytes):
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, nbytes + 4096, dtype=np.uint8)).cuda()
    dst = torch.full((nbytes + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    HN.moe_stream_probe(src, dst, nbytes, HN.MOE_PROBE_COPY)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert bool((dst[nbytes:] == 0xA5).all()), "the copy wrote past its end"


@pytest.mark.parametrize("mode", [HN.MOE_PROBE_READ_CACHED, HN.MOE_PROBE_READ_STREAM],
                         ids=["cached", "stream"])
@pytest.mark.parametrize("nbytes", [16, 16384, 16384 * 5 + 4096, (1 << 24) + 16])
def test_read_counts_all_ones_vectors(mode, nbytes):
    rng = np.random.default_rng(nbytes + mode)
    words = rng.integers(0, 2 ** 31, (nbytes + 64) // 4, dtype=np.uint32)
    vec = words.reshape(-1, 4)
    n_vec = nbytes // 16
    planted = np.unique(rng.integers(0, n_vec, min(n_vec, 37)))
    vec[planted] = 0xFFFFFFFF
    vec[n_vec:] = 0xFFFFFFFF  # past the sweep: must not be counted
    src = torch.from_numpy(words.view(np.uint8)).cuda()
    cnt = torch.zeros(2, dtype=torch.int32, device="cuda")
    HN.moe_stream_probe(src, cnt, nbytes, mode)
    torch.cuda.synchronize()
    assert int(cnt[0].item()) == planted.size
    assert int(cnt[1].item()) == 0
