import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library with device 0 initialised; fails (not skips) when
    the library is missing, so a GPU run can never pass on a fallback."""
    import torch
    from int8_w8a8_quantized_amd import lib as w8lib
    assert torch.cuda.is_available(), "gpu tests need a GPU"
    L = w8lib.load()
    w8lib.init(0)
    return L
