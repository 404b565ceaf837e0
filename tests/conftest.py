import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests of the HIP path")
    config.addinivalue_line("markers", "slow: long CPU statistics tests")


def pytest_runtest_setup(item):
    # A GPU test on a machine without a GPU fails loudly instead of skipping,
    # so a box whose GPU is not visible cannot pass the GPU tier silently.
    if "gpu" in item.keywords:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("GPU test selected but torch.cuda.is_available() is False")
        print(f"\n[gpu-test] {item.nodeid}", flush=True)


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (built here if nothing is built yet), or the
    one DPNORM_TEST_LIB names (the host-layer build under sanitizers)."""
    from sample_grad_norms_amd import _lib
    other = os.environ.get("DPNORM_TEST_LIB")
    if other:
        return _lib.load(other)
    if not os.path.exists(_lib.LIB_PATH):
        from sample_grad_norms_amd import build as _build
        _build.build_library()
    return _lib.load()
