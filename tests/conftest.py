import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.lib()


@pytest.fixture
def hook():
    """Sets libfq's test hook (fq_test_hook) for one test and restores the defaults after it."""
    import w4a4_integer_gemm_amd as fq
    fq.fq_test_hook("")
    yield fq.fq_test_hook
    fq.fq_test_hook("")
