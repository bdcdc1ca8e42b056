import functools
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@functools.lru_cache(maxsize=None)
def oracle_codebook(d: int, bits: int):
    """Float32 codebook from the oracle's Lloyd iteration (cached per session)."""
    import numpy as np
    import oracle
    return oracle.lloyd_max(d, bits).astype(np.float32)


@pytest.fixture(scope="session")
def cb():
    return oracle_codebook
