import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """GPU tests fail loudly (not skip) when run without a GPU only if the user
    asked for them with -m gpu; an unfiltered CPU run skips them."""
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    markexpr = config.getoption("-m") or ""
    if have_gpu or "gpu" in markexpr.replace("not gpu", ""):
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
