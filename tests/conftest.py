import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """Worst bf16 output error each parity test observed (against the oracle)."""
    helpers = sys.modules.get("tests.helpers")
    obs = getattr(helpers, "OBSERVED", None) if helpers else None
    if not obs:
        return
    terminalreporter.write_line("parity errors (worst rel-L2, worst max-abs, comparisons):")
    for test, (err, mx, n) in sorted(obs.items()):
        terminalreporter.write_line("  %-90s %.3e %.3e %d" % (test, err, mx, n))
