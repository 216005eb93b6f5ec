import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-size case (full workload shapes)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Observed parity errors: max abs error and the fraction of the
    per-element bar each comparison used (the largest first)."""
    try:
        from helpers import ERROR_LOG
    except ImportError:
        return
    if not ERROR_LOG:
        return
    tr = terminalreporter
    tr.section("parity errors (max |err|, share of the per-element bar)")
    for what, dtype, err, used in sorted(ERROR_LOG, key=lambda r: -r[3]):
        tr.write_line(f"{used:6.3f}  {err:.3e}  {dtype:4s}  {what}")
