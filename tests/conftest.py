import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_POOL = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The oracle's worker processes are started here, before anything in this process
    # touches a GPU (collection below asks torch whether one is visible): they are
    # spawned interpreters that hold no GPU state, and the GPU tests later only send
    # them inputs.  ORACLE_PROCESSES=1 runs the oracle in this process instead (for
    # runs under a profiler, whose preloaded library initialises the GPU at start).
    global _POOL
    import oracle

    if oracle.oracle_processes() > 1:
        _POOL = oracle.head_pool()
        oracle.set_default_pool(_POOL)


def pytest_unconfigure(config):
    global _POOL
    if _POOL is not None:
        import oracle

        oracle.set_default_pool(None)
        _POOL.terminate()
        _POOL.join()
        _POOL = None


def pytest_collection_modifyitems(config, items):
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
