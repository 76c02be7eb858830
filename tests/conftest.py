import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound through its C ABI.  Fails (not skips) when a GPU
    is present but the library is missing: the HIP path must be the one run."""
    if not _gpu_available():
        pytest.skip("no GPU visible")
    import selective_state_space_81_amd as ms
    ms.load()  # raises if libmsscan.so is absent
    return ms
