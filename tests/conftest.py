import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Lines the parity tests print with their measured errors (one JSON record each).  pytest keeps the
# captured output of passing tests out of the terminal, so they are collected here and printed again in
# the terminal summary: the run's log then carries every measured margin, also under -q.
RECORD_TAGS = ("PARITY ", "SPLIT ", "COVER ", "DENSE ", "DIAG ", "POOLED ", "PRED ", "SCALE ", "NOALLOC ",
               "SELECT ")
_records = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload check (minutes of host time)")


def pytest_runtest_logreport(report):
    if report.when != "call":
        return
    for line in report.capstdout.splitlines():
        if line.startswith(RECORD_TAGS):
            _records.append(line)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not _records:
        return
    terminalreporter.section("measured errors of the parity cases")
    for line in _records:
        terminalreporter.write_line(line)
