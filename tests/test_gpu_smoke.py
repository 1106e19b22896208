"""The build's smoke entry point, run as a GPU test so that it is checked
whenever the GPU suite runs: one decode GEMV, one MFMA GEMM, one grouped call
with the weighted sum and one producer-fed small batch, each against the CPU
oracle."""
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_smoke_entry_point():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import __graft_entry__

    __graft_entry__.smoke()
