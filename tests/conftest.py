import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture
def mrr_env():
    """Sets libmrr's MRR_* environment overrides for one test.  The library
    reads them at load time and on mrr_reload_env(); the fixture calls it
    after every change and again after restoring the environment, so an
    override never outlives its test (not even a failing one)."""
    import allreduce_reduction_nranks_amd as mrr
    saved = {}

    def set_override(name, value):
        if name not in saved:
            saved[name] = os.environ.get(name)
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = str(value)
        mrr.mrr_reload_env()

    yield set_override
    for name, value in saved.items():
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = value
    mrr.mrr_reload_env()
