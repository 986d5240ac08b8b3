import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The GPU library's Python binding.  On a machine with a GPU this must load:
    a missing or broken HIP library fails the test instead of skipping it."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import dense_tiled_gemm_04_amd as g
    g.load()  # raises if the shared library is missing
    return g
