import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; skips when no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_kv_prefix_amd as fb
    fb.load()          # raises if the shared library is missing: no silent fallback
    return fb


@pytest.fixture(autouse=True)
def _guard_bands():
    """Checks, after each test, the canary regions around the buffers the test cut out with
    tests.gpu_util.guarded (a no-op for tests that use none)."""
    from tests import gpu_util
    gpu_util.GUARDS.clear()
    yield
    gpu_util.check_guards()
