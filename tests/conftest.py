import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_ready():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # A GPU test on a machine without a GPU is reported as skipped, not failed.
    # When GPU tests were asked for explicitly (-m gpu) they must run and fail
    # loudly without a GPU; otherwise they are skipped on a GPU-less machine.
    if _gpu_ready() or config.getoption("markexpr", "").strip() == "gpu":
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
