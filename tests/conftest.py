import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path through the C ABI)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than ~20 s")


@pytest.fixture(scope="session")
def cfg1():
    import synth
    return synth.config1()


@pytest.fixture(scope="session")
def cfg1_packed(cfg1):
    import oracle
    return oracle.pack_kv_4bit(cfg1.K, cfg1.V, cfg1.n // 32)
