import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0; GPU tests fail (not skip) when either is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch sees no GPU")
    from decode_attention_03_amd import fd

    dev = torch.device("cuda:0")
    # the HIP runtime and the device context come up before any test draws
    # inputs (the input generator runs a thread pool)
    torch.cuda.init()
    torch.empty(1, device=dev)
    torch.cuda.synchronize(dev)
    fd.library()  # raises if libfd.so is missing, stale or fails to load
    return dev
