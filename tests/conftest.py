import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    # every error the GPU parity tests measured, with its bound (a passing
    # run's log then shows the margins, not just a pass)
    try:
        import parity_log
    except ImportError:
        return
    lines = parity_log.summary_lines()
    if lines:
        terminalreporter.section("parity errors against the fp64 oracle")
        for line in lines:
            terminalreporter.write_line(line)
