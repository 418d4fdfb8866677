import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; on a CPU-only host they are skipped with a reason
    # instead of failing, so `-m "not gpu"` and a bare run behave the same here.
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
    # the errors the parity tests measured against the oracle, one line per comparison, so that a
    # quiet run's summary still states them
    h = sys.modules.get("harness")
    lines = getattr(h, "PARITY", None)
    if lines:
        terminalreporter.section("measured error against the oracle")
        for line in lines:
            terminalreporter.write_line(line)
