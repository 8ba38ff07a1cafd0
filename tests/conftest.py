import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; on a CPU-only host they are
    # reported as skipped instead of failing on a missing device.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def ora():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def syn():
    import synth
    synth.cpu_lib()
    return synth
