"""The smoke check of __graft_entry__ runs green on the GPU."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke():
    import __graft_entry__
    __graft_entry__.smoke()
