"""CU-mask construction (host only): every XCD keeps compute units under
either reading of the mask bits, and the two slices are complementary."""
import pytest

from combine_fp32_router_amd.custreams import mask_words


@pytest.mark.parametrize("quarters", [1, 2, 3])
def test_masks_cover_every_xcd_and_complement(quarters):
    ncu, xcds = 256, 8
    lo = mask_words(ncu, quarters)
    hi = mask_words(ncu, quarters, upper=True)
    assert len(lo) == len(hi) == ncu // 32
    bits_lo = [w * 32 + b for w, word in enumerate(lo) for b in range(32) if word >> b & 1]
    bits_hi = [w * 32 + b for w, word in enumerate(hi) for b in range(32) if word >> b & 1]
    assert len(bits_lo) == ncu * quarters // 4
    assert set(bits_lo).isdisjoint(bits_hi) and len(bits_lo) + len(bits_hi) == ncu
    for bits in (bits_lo, bits_hi):
        assert {b % xcds for b in bits} == set(range(xcds))    # interleaved reading
        assert {b // 32 for b in bits} == set(range(xcds))     # blocks-of-32 reading


def test_mask_rejects_bad_arguments():
    with pytest.raises(ValueError):
        mask_words(256, 4)
    with pytest.raises(ValueError):
        mask_words(250, 2)
