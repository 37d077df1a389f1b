import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The HIP library through its Python binding (GPU tests only)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import w4a16_decode_gemv_amd as w4

    w4.load()  # raises if the built library is missing
    return w4
