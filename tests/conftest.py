import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI")
    config.addinivalue_line("markers", "slow: larger parity cases")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    try:
        from tests.gpu_support import OBSERVED
    except Exception:  # pragma: no cover
        return
    if not OBSERVED:
        return
    terminalreporter.write_sep("-", "largest observed errors against the oracle")
    for name in sorted(OBSERVED):
        terminalreporter.write_line(f"{name}: {OBSERVED[name]:.3e}")
