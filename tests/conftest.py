import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle


_FULL_X = {}


@pytest.fixture(scope="session")
def full_tokens():
    """full_tokens(cfg): the seeded X of a workload at its full N (generated once
    per session; about 1 GiB for the headline)."""
    def get(cfg):
        if cfg.name not in _FULL_X:
            _FULL_X[cfg.name] = cfg.x_rows(0)
        return _FULL_X[cfg.name]
    return get
