import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def da():
    """The HIP library binding; GPU tests fail loudly if it is not built."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import sparse_kv_cache_gqa_amd as pkg
    pkg.load()  # raises if libda.so is missing
    return pkg
