import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The product binding with its HIP library loaded; fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    import scaled_dot_product_03_amd as sdpa
    sdpa.load()          # raises if the shared library is absent
    return sdpa
