import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


@pytest.fixture(autouse=True)
def _device_index_checks(request):
    """With SPECVERIFY_LIBRARY naming the build with device-side index checks, every GPU
    test must end with no failed check."""
    if request.node.get_closest_marker("gpu") is None or not os.environ.get("SPECVERIFY_LIBRARY"):
        yield
        return
    import torch

    import device_draft_verification_specverify_amd as sv

    if sv.check_count(reset=True) is None:
        yield
        return
    yield
    torch.cuda.synchronize()
    n = sv.check_count(reset=True)
    assert n == 0, f"{n} failed device-side index checks"


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load
