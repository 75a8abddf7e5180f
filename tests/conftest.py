import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C-ABI")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Worst |gpu - oracle| / bound per test file of the GPU parity tests."""
    try:
        from gpu_case import RATIOS
    except Exception:
        return
    if RATIOS:
        terminalreporter.write_sep("-", "worst err/bound per file")
        for f in sorted(RATIOS):
            terminalreporter.write_line("%s: %.4f" % (f, RATIOS[f]))
