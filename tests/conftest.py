import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs; minutes of CPU work")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every GPU output comparison of the run: its largest error against the oracle
    and how many elements needed the P-code flip allowance (capped at the bar)."""
    try:
        from _parity import RECORDS
    except ImportError:
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("output parity against the oracle")
    n_exc = sum(r[3] for r in RECORDS)
    tr.write_line(f"{len(RECORDS)} comparisons, {sum(r[1] for r in RECORDS)} elements; "
                  f"largest error {max(r[2] for r in RECORDS):.3e}; "
                  f"{n_exc} element(s) excused by the flip allowance"
                  + (f" (largest excess over the bar {max(r[4] for r in RECORDS):.2e})" if n_exc else ""))
    for what, n, e, k, x in RECORDS:
        tr.write_line(f"  {what}: {n} elements, max err {e:.2e}" + (f", {k} excused (excess {x:.2e})" if k else ""))
