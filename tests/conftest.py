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


def pytest_collection_modifyitems(config, items):
    # GPU tests are selected with -m gpu; when they are selected on a machine
    # without a GPU they fail loudly rather than silently passing.
    if _gpu_available():
        return
    for item in items:
        if "gpu" in item.keywords and config.getoption("-m") != "gpu":
            item.add_marker(pytest.mark.skip(reason="no GPU on this machine"))


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle._lib()
    return oracle
