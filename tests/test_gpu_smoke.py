"""The build entry point's smoke check (one small dispatch -> stand-in expert
-> combine round trip on cuda:0, compared with the oracle) runs under pytest
too, not only when the entry point is called directly."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    import __graft_entry__ as g
    g.smoke()
