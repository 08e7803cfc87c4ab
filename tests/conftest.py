import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library through its Python binding, on cuda:0."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import invariant_amd as bi
    bi.load()                     # raises if the HIP library is missing
    return bi
