import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


@pytest.fixture(scope="session")
def lib():
    """The HIP library binding; GPU tests only."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import loftq_qlora_initialization_amd as lq
    return lq


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU test on the real stderr before it runs, so a run that dies mid-test says where."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
