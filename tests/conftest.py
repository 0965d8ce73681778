import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: full-size workload parity (minutes on the host)")


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _have_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible: the HIP path cannot run here")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity report the GPU tests collected: per configuration, the
    rows compared, the rows and blocks whose GPU support differs from the
    oracle's in boundary-flagged blocks only, and the largest output errors."""
    try:
        from parity_helpers import REPORT
    except ImportError:
        return
    if not REPORT:
        return
    terminalreporter.write_sep("-", "parity report (GPU vs fp64 oracle)")
    for cfg, fields in REPORT:
        terminalreporter.write_line(f"{cfg}: " + ", ".join(
            f"{k} {v:.3e}" if isinstance(v, float) else f"{k} {v}" for k, v in fields.items()))
