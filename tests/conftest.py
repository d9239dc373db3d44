import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a 'key v1 v2 ...' fixture; '#' lines are comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (MI355X); run with -m gpu")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def bgb_gpu():
    """The device library through its Python binding; fails loudly if missing."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import bit_gemm_binarize_amd as bgb
    bgb.load()  # raises if libbgb.so is not built
    return bgb
