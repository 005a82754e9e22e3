import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The worst achieved relative error of each parity test (fp32 paths)."""
    try:
        from tests import parity
    except Exception:
        return
    if not parity.ACHIEVED:
        return
    terminalreporter.write_line("worst achieved relative errors (test, quantity, error):")
    for (test, kind), v in sorted(parity.ACHIEVED.items()):
        terminalreporter.write_line(f"  {test} {kind} {v:.2e}")
