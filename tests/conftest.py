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
def mk():
    """The ctypes binding with its library loaded; GPU tests only."""
    if not gpu_available():
        pytest.fail("GPU test collected without a GPU (select with -m 'not gpu')")
    from communication_gemm_persistent_amd import mk as binding
    binding.load()
    return binding
