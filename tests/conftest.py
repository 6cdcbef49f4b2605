import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large shapes, minutes of work")


def max_rel_err(a, b):
    """max|a - b| / max|b| over a whole tensor (the graded error measure)."""
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.abs(b).max() if b.size else 0.0
    num = np.abs(a - b).max() if b.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


@pytest.fixture
def rel_err():
    return max_rel_err


# Largest error seen per (group, tensor) over the cases a run checked; printed at the end
# of every run (also with -q, and when every test passes) so the parity margins of a
# GPU run are visible in its log.
_PARITY = {}


def record_parity(group, **errs):
    d = _PARITY.setdefault(group, {})
    for k, v in errs.items():
        d[k] = max(d.get(k, 0.0), float(v))


def pytest_terminal_summary(terminalreporter):
    if not _PARITY:
        return
    terminalreporter.write_line("parity summary (largest max|a-b|/max|b| over the checked cases):")
    for group in sorted(_PARITY):
        errs = _PARITY[group]
        terminalreporter.write_line(f"  {group}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
