import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The product binding, loaded for GPU tests; fails loudly when missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    import gated_deltanet_tree_verify_amd as g
    g.load()
    return g
