import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X); calls the HIP library")


@pytest.fixture(scope="session")
def O():
    import oracle
    if not os.path.exists(oracle.lib_path()):
        oracle.build(force=False)
    return oracle.Oracle()


def has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture
def progress(request):
    """A function that prints a line at once, past pytest's output capture (long tests show
    that they are working)."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def emit(msg: str) -> None:
        with capman.global_and_fixture_disabled():
            sys.stderr.write(msg + "\n")
            sys.stderr.flush()
    return emit
