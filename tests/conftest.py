import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload checks")


@pytest.fixture(scope="session")
def rf_gpu():
    """The HIP binding, on a machine with a GPU. Fails (not skips) if the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import online_softmax_attention_pass_amd as rf
    rf.load()  # raises if the built library is absent
    return rf
