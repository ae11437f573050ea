import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload cases")


def pytest_collection_modifyitems(config, items):
    # GPU tests are selected with -m gpu; without a GPU they are skipped rather than failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # names the case before any GPU work starts, so a run that dies mid-test says which one
    if "gpu" in request.keywords:
        print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
