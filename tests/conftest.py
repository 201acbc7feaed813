import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large oracle comparison")


def pytest_terminal_summary(terminalreporter):
    """Worst measured parity errors of the session, per compared quantity."""
    parity = sys.modules.get("parity") or sys.modules.get("tests.parity")
    if parity is None or not parity.WORST:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity: largest |gpu - oracle| per quantity (max, mean; tolerance)")
    for (what, dtype), (mx, mean, n) in sorted(parity.WORST.items()):
        tmax, tmean = parity.TOL[dtype]
        tr.write_line(f"{what:<28} {dtype:<5} max {mx:.3e} (tol {tmax:g})  mean {mean:.3e} "
                      f"(tol {tmean:g})  over {n} comparisons")
