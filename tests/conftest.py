import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    require = os.environ.get("MMDIT_REQUIRE_GPU") == "1"
    for item in items:
        if "gpu" in item.keywords:
            if require:
                item.add_marker(pytest.mark.xfail(reason="no GPU but MMDIT_REQUIRE_GPU=1", strict=True, run=False))
            else:
                item.add_marker(pytest.mark.skip(reason="no GPU in this process"))
