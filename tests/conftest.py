"""Shared test configuration.

Marker ``gpu``: the test needs an MI355X (gfx950) and the built HIP library.
The CPU suite runs with ``-m "not gpu"``.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libkvarn.so")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def dev():
    """The GPU device; GPU tests fail loudly when the HIP library cannot load."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible to this process")
    from kv_cache_quantization_x128_amd import kvarn

    kvarn.load()  # raises if libkvarn.so is missing or stale
    return torch.device("cuda:0")
