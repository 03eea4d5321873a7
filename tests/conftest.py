import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.lib()  # builds liboracle.so on first use if absent
    return o


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def fp8q():
    """The HIP library binding; GPU tests fail loudly if it cannot be used."""
    if not _gpu_available():
        pytest.fail("GPU test selected but no HIP device is visible")
    import fp8_fine_grained_x128_amd as f
    return f
