import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """How many rows each full-size parity case checked (tests/gpu_util.RECORDS)."""
    gu = sys.modules.get("tests.gpu_util")
    if gu is None or not getattr(gu, "RECORDS", None):
        return
    terminalreporter.section("full-size parity: rows value-checked against the fp64 oracle")
    for line in gu.RECORDS:
        terminalreporter.write_line(line)
