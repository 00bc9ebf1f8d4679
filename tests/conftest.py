import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: full-size model runs (minutes)")


def pytest_collection_modifyitems(config, items):
    # A test module marked gpu is skipped here if no GPU is visible, unless the
    # caller asked for gpu tests explicitly (then a missing GPU is an error).
    markexpr = config.getoption("-m") or ""
    want_gpu = "gpu" in markexpr and "not gpu" not in markexpr
    if want_gpu:
        return
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
