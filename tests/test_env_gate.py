"""CPU check of the GPU-test gate: without a GPU, GPU tests are skipped, and
with MMDIT_REQUIRE_GPU=1 they fail (a machine meant to run them cannot pass
by skipping)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# one small GPU test, selected by node id
TARGET = "tests/test_gpu_step.py::test_rope_table_matches_oracle"


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def _run(require: bool):
    env = dict(os.environ)
    env.pop("MMDIT_REQUIRE_GPU", None)
    if require:
        env["MMDIT_REQUIRE_GPU"] = "1"
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", TARGET], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(_gpu_visible(), reason="checks the behaviour without a GPU")
def test_gpu_tests_skip_without_gpu():
    r = _run(False)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "1 skipped" in r.stdout


@pytest.mark.skipif(_gpu_visible(), reason="checks the behaviour without a GPU")
def test_require_gpu_makes_gpu_tests_fail():
    r = _run(True)
    assert r.returncode == 1, r.stdout + r.stderr
    assert "1 failed" in r.stdout and "MMDIT_REQUIRE_GPU=1" in r.stdout
