import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")
    config.addinivalue_line("markers", "oracle_pool: uses the forked oracle worker pool")


def pytest_unconfigure(config):
    import oracle_pool
    oracle_pool.stop()


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a CPU-only host they are skipped, never run on a fallback.
    # Counting devices does not initialise the GPU, so the oracle worker pool can still be forked
    # here, before any test runs, when a selected test wants it.
    try:
        import torch
        has_gpu = torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        if any(it.get_closest_marker("oracle_pool") for it in items):
            import oracle_pool
            oracle_pool.start()
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
