import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libpkv.so")
    config.addinivalue_line("markers", "slow: large inputs (full-size workloads)")


def pytest_collection_modifyitems(config, items):
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst err/allowed of every parity family that ran (1.0 = at the gate)."""
    try:
        import _margins
    except ImportError:  # pragma: no cover
        return
    if not _margins.WORST:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity margins: worst err/allowed per test family (gate = 1.0)")
    for fam in sorted(_margins.WORST):
        ratio, case, err, ref = _margins.WORST[fam]
        tr.write_line(f"{ratio:7.3f}  {fam}  (case {case}: max|err| {err:.2e}, max|ref| {ref:.2e})")
