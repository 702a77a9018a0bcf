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


def _require_gpu() -> bool:
    return os.environ.get("MMDIT_REQUIRE_GPU") == "1"


def pytest_collection_modifyitems(config, items):
    # Without a GPU, GPU tests are skipped, unless MMDIT_REQUIRE_GPU=1 asks
    # for them to run: then each one fails (see pytest_runtest_call below).
    if _gpu_available() or _require_gpu():
        return
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(pytest.mark.skip(reason="no GPU in this process"))


@pytest.hookimpl(tryfirst=True)
def pytest_runtest_call(item):
    """With MMDIT_REQUIRE_GPU=1 a GPU test fails when no GPU is visible, so a
    machine that should run them cannot pass by skipping them."""
    if item.get_closest_marker("gpu") is not None and _require_gpu() and not _gpu_available():
        pytest.fail("MMDIT_REQUIRE_GPU=1 but no GPU is visible to this process")
