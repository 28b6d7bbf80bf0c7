import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # Load what is built; build only when nothing is.
    from oracle import build as obuild
    if not os.path.exists(obuild.LIB_PATH):
        obuild.build()
    try:
        from rope_partial_inplace_amd import build as lbuild
    except ImportError:
        return
    if not os.path.exists(lbuild.LIB_PATH):
        lbuild.build()


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU (run with -m 'not gpu')")
    return torch.device("cuda:0")
