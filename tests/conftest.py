import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "large: full-size workload (minutes of CPU oracle time)")


def pytest_terminal_summary(terminalreporter):
    """One line with the worst accuracy margin of every checked output:
    ratio = err / (2 floor) (the criterion passes at <= 1), the same against
    the unrounded floor, and the gradient rel-L2."""
    import json
    from tests import criteria
    if criteria.RECORDS:
        terminalreporter.write_line("CRITERIA_SUMMARY " + json.dumps(criteria.summary(),
                                                                     separators=(",", ":")))
