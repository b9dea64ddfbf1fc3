import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (still part of the default suites)")


@pytest.fixture
def progress(capsys):
    """A progress printer for long tests: each line goes past pytest's capture to the real
    stdout (flushed), and is appended to the file MPSTEP_PROGRESS_LOG names, if set, so that
    a long test is seen to be alive while it runs."""
    log = os.environ.get("MPSTEP_PROGRESS_LOG")

    def say(*a):
        line = " ".join(str(x) for x in a)
        with capsys.disabled():
            print(line, flush=True)
        if log:
            try:
                with open(log, "a") as f:
                    f.write(line + "\n")
            except OSError:
                pass
    return say


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.lib()
