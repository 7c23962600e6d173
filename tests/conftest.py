import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (full-size oracle work)")
    # The full-size parity tests run the oracle in worker processes forked
    # from a server process; it must start before anything initialises the
    # GPU (collection below asks torch whether a GPU is visible).  Counting
    # devices does not initialise them.
    if "not gpu" in (config.getoption("markexpr", "") or ""):
        return
    try:
        import torch

        if torch.cuda.device_count() > 0:
            import oracle_jobs

            oracle_jobs.start_server()
    except ImportError:  # pragma: no cover
        pass


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; without one they are skipped, never faked.
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
