import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) where no GPU is visible, so the CPU
    # tier `-m "not gpu"` and a plain run on a CPU host both stay green.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture
def knob():
    """knob(name, value) forces a library path (dq_set_knob) for one test;
    every knob it touched is restored afterwards, pass or fail."""
    import kv_cache_entropy_amd as dq
    old = {}

    def set_(name, value):
        if name not in old:
            old[name] = dq.get_knob(name)
        dq.set_knob(name, value)

    yield set_
    for name, value in old.items():
        dq.set_knob(name, value)
