import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """Skip cleanly when no GPU is visible; otherwise return the loaded HIP library binding."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import block_scaled_fp4_amd as fp4
    fp4.load()  # raises if the native library is missing: no silent fallback
    return fp4
