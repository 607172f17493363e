import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# The mutation tests run the pin suite against a planted-mistake copy of the oracle package.
if os.environ.get("ADAMW4_ORACLE_PKG"):
    sys.path.insert(0, os.environ["ADAMW4_ORACLE_PKG"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle
