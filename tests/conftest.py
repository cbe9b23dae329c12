import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line(
        "markers",
        "gpu: needs an MI355X (gfx950); calls the HIP library through its C ABI")


@pytest.fixture(scope="session")
def dev():
    """cuda:0 with the HIP library loaded; skips only when no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import quant_gemm_amd as mq
    mq.load()          # raises if libmq.so is missing: no fallback path exists
    return torch.device("cuda:0")
