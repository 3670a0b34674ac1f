import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _built_oracle():
    import oracle
    if not os.path.exists(oracle._LIB):
        oracle.build()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_gist_amd as gsa
    gsa.lib()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")
