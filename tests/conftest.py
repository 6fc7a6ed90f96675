import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """The largest attention error (relative to the reference's largest
    value) of each test that compared attention outputs, worst first."""
    helpers = sys.modules.get("helpers")
    margins = getattr(helpers, "MARGINS", None)
    if not margins:
        return
    worst = {}
    for test, e in margins:
        worst[test] = max(worst.get(test, 0.0), e)
    terminalreporter.write_sep("-", f"attention parity: largest relative error per test (bar {helpers.TOL:.0e})")
    for test, e in sorted(worst.items(), key=lambda kv: -kv[1]):
        terminalreporter.write_line(f"{e:.2e}  {e / helpers.TOL:5.1%} of the bar  {test}")
