import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """Fails loudly (never skips) when a GPU test runs without a GPU or without the library."""
    import torch
    assert torch.cuda.is_available(), "GPU test run on a machine without a GPU"
    import spatial_temporal_sparse_amd as svg  # raises if libsvg.so is missing
    return svg
