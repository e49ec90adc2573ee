import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes on the CPU side)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The C-ABI library with a live GPU; GPU tests fail (not skip) if the
    library is missing, so a missing build can never pass silently."""
    import torch

    from deltanet_delta_rule_chunk_amd import binding

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return binding.load()
