import os
import sys
import zlib

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _rng_per_test(request):
    """A test module's ``RNG`` (the oracle pins draw their inputs from one)
    is reseeded from the test's own id before each test, so the inputs do
    not depend on which tests ran before it in the same process (as they
    would when tests are spread over several worker processes)."""
    mod = request.module
    if isinstance(getattr(mod, "RNG", None), np.random.Generator):
        mod.RNG = np.random.default_rng(zlib.crc32(request.node.nodeid.split("::", 1)[-1].encode()))
