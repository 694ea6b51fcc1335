import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
for p in (ROOT, ROOT / "tests"):
    if str(p) not in sys.path:
        sys.path.insert(0, str(p))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configurations (tens of seconds each)")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_tests_need_a_gpu(request):
    """GPU tests are skipped only where there is no GPU at all; on a GPU machine a missing
    library makes them fail loudly (the binding raises)."""
    if request.node.get_closest_marker("gpu"):
        import torch
        if not torch.cuda.is_available():
            pytest.skip("no GPU in this machine")
