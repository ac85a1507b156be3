import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large workload, minutes of CPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, loaded through its ctypes binding."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conditional_draft_tree_depth_amd import _lib
    return _lib.load()
