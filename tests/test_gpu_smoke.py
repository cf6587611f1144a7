"""The round-trip check __graft_entry__.smoke() runs: one small layer on
row-major and packed weights against the oracle (kept in the GPU suite so
that a kernel change which breaks it is caught by pytest too)."""
import os
import sys

import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_smoke_entry_point():
    if HERE not in sys.path:
        sys.path.insert(0, HERE)
    import __graft_entry__
    __graft_entry__.smoke()
