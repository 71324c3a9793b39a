import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library bound through its Python wrapper; fails loudly without a GPU."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import int4_weight_only_gptq_amd as qg

    qg.load()
    return qg
