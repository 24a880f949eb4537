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
    """Every GPU output comparison of the run: its largest error against the oracle,
    that error's largest ratio to the element's own bound (a ratio above 1 fails),
    and how many elements needed a code-flip allowance (capped; the excess is
    absolute for outputs, relative to the term magnitude for gradients)."""
    try:
        from _parity import RECORDS
    except ImportError:
        return
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("output parity against the oracle")
    worst = max(RECORDS, key=lambda r: r[6])
    tr.write_line(f"{len(RECORDS)} comparisons, {sum(r[1] for r in RECORDS)} elements; "
                  f"largest error {max(r[2] for r in RECORDS):.3e}; largest error / per-element bound "
                  f"{worst[6]:.3f} ({worst[0]}); "
                  f"{sum(r[3] for r in RECORDS)} element(s) excused by a code-flip allowance")
    for what, n, e, k, x, unit, ratio in RECORDS:
        tr.write_line(f"  {what}: {n} elements, max err {e:.2e}, err/bound {ratio:.3f}"
                      + (f", {k} excused (excess {x:.2e}{unit})" if k else ""))
