import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU time)")


@pytest.fixture(scope="session")
def root():
    return ROOT


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per test file: how many Top-P sets matched the oracle exactly
    and how many were accepted under the bin-edge or the mass-margin rule."""
    parity = sys.modules.get("parity")
    stats = getattr(parity, "SET_STATS", None)
    if not stats:
        return
    for f, c in sorted(stats.items()):
        terminalreporter.write_line(f"Top-P sets {f}: {c['exact']} exact, {c['edge']} edge-tolerated, "
                                    f"{c['margin']} margin-tolerated")
