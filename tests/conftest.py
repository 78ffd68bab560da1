import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases")


def pytest_collection_modifyitems(config, items):
    # GPU tests are only meaningful on a box with a GPU; on a CPU-only host they are skipped
    # rather than failing, so `-m "not gpu"` and a bare run both stay green here.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


class GemmForce:
    """The library's test-only GEMM override (ttl_set_gemm_override), set field by field."""

    def __init__(self):
        from tensor_transformer_linear_amd import ttl
        self._ttl = ttl
        self.state = dict(kernel="auto", splits=0, plan_cus=0, trace=False)

    def set(self, **kw):
        self.state.update(kw)
        self._ttl.set_gemm_override(**self.state)

    def reset(self):
        self.state = dict(kernel="auto", splits=0, plan_cus=0, trace=False)
        self._ttl.set_gemm_override()


@pytest.fixture
def gemm_force():
    """Forces GEMM kernel choices for one test; the choice by shape is restored afterwards."""
    f = GemmForce()
    f.reset()
    yield f
    f.reset()
