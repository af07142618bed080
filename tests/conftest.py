import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Under pytest-xdist every worker would start one OpenMP thread per core for
# the oracle's (tiny) CPU calls, and spinning idle threads oversubscribe the
# host by the worker count (a 30 s suite then takes over ten minutes).  One
# thread per worker unless the caller chose otherwise; set before libgomp
# reads it, i.e. before the oracle library is loaded.
if os.environ.get("PYTEST_XDIST_WORKER"):
    os.environ.setdefault("OMP_NUM_THREADS", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import oracle
    return oracle.load()
