import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built libqgguf.so")
    config.addinivalue_line("markers", "big: full-size workload (hundreds of MB of weights)")


def pytest_collection_modifyitems(config, items):
    if any(item.get_closest_marker("gpu") for item in items):
        try:
            import torch
            have_gpu = torch.cuda.is_available()
        except Exception:
            have_gpu = False
        if not have_gpu:
            skip = pytest.mark.skip(reason="no GPU visible")
            for item in items:
                if item.get_closest_marker("gpu"):
                    item.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
