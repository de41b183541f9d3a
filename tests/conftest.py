import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

# The oracle's process pool forks its workers from a server started now,
# before any test initialises the GPU.
import oracle_side  # noqa: E402

oracle_side.start()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A run without "-m gpu" on a machine without a GPU must not fail on GPU tests.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    # Under an explicit "-m gpu" nothing is skipped: a GPU run without a GPU fails.
    if has_gpu or "gpu" in (config.option.markexpr or "").replace("not gpu", ""):
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
