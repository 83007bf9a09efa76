import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

GOLDEN = os.path.join(TESTS, "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture
def golden():
    return golden_rows


@pytest.fixture(autouse=True)
def _fresh_oracle_counts():
    """The oracle memoizes step counts per argument tuple; a test that plants a
    mistake in a replay must not see counts cached from the correct one."""
    from oracle import cost
    cost._COUNTS.clear()
    yield
    cost._COUNTS.clear()
