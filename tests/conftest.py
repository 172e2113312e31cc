import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is present; the CPU suite never touches HIP.
    gpu_ok = None
    for item in items:
        if "gpu" in item.keywords:
            if gpu_ok is None:
                try:
                    import torch
                    gpu_ok = torch.cuda.is_available()
                except Exception:  # pragma: no cover
                    gpu_ok = False
            if not gpu_ok:
                item.add_marker(pytest.mark.skip(reason="no GPU in this environment"))
