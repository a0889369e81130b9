import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not _has_gpu():
        pytest.skip("no GPU")
    import torch
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """With PKV_PARITY_LOG set, write every parity comparison's margins there."""
    path = os.environ.get("PKV_PARITY_LOG")
    if not path:
        return
    mod = sys.modules.get("gpu_common")
    if mod is not None and mod.PARITY_LOG:
        mod.write_parity_log(path)
