import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload parity (minutes on the CPU oracle)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, on a machine that has a GPU. Fails loudly otherwise."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import linear_attention_ssm_amd as gdn
    return gdn
