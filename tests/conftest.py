import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def import_zs():
    """The library's binding; on a checkout where the library is not built
    yet, build it first (hipcc cross-compiles gfx950 code without a GPU)."""
    import importlib
    import subprocess
    try:
        return importlib.import_module("fsdp_sharded_mixed_flatten_amd")
    except ImportError:
        subprocess.run([sys.executable, os.path.join(ROOT, "fsdp_sharded_mixed_flatten_amd", "build.py")],
                       check=True)
        return importlib.import_module("fsdp_sharded_mixed_flatten_amd")


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


@pytest.fixture(autouse=True)
def _release_device_memory():
    """After each test: unbind whatever multi-tensor workspace it left bound
    (the binding keeps every bound tensor alive until then), and hand the
    blocks torch's caching allocator holds back to the device, so the next
    test's free-memory check sees them (the full-size tests need nearly the
    whole of it)."""
    yield
    zs = sys.modules.get("fsdp_sharded_mixed_flatten_amd")
    bound = getattr(zs, "_bindings", None) if zs is not None else None
    if bound:
        for ws, _refs in list(bound.values()):
            try:
                zs.zs_multi_unbind(ws)
            except Exception:  # pragma: no cover - a failed test may leave the device unusable
                pass
        bound.clear()
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        import gc
        gc.collect()
        torch.cuda.empty_cache()
