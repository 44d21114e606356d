import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


@pytest.fixture(scope="session")
def oracle_pool():
    """A process pool running the float64 oracle head by head (every host
    core), for full-size comparisons; shared by the whole session."""
    from oracle.pool import OraclePool
    pool = OraclePool()
    yield pool
    pool.close()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
