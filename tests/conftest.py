import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Near-tie counts of the GPU parity cases (allocation mismatches inside
    the 1e-6 window), one line per case."""
    from tests import parity_util
    if parity_util.REPORT:
        terminalreporter.section("GPU vs oracle: near ties per case")
        for line in parity_util.REPORT:
            terminalreporter.write_line(line)
