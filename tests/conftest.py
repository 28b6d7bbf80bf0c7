import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _module_from_file(name: str, path: str):
    """Load a build script by path: importing it through its package would run the package's
    __init__, which refuses to import before its library exists."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # Test what is built, and only if it was built from the sources as they are now: a
    # missing or stale library is rebuilt on a machine without a GPU; where there is a GPU the
    # session stops instead (libraries are built before a GPU run, never inside one).
    on_gpu_host = os.path.exists("/dev/kfd")
    for name, rel in (("_oracle_build", ("oracle", "build.py")),
                      ("_rope_lib_build", ("rope_partial_inplace_amd", "build.py"))):
        if name == "_oracle_build" and os.environ.get("ROPE_ORACLE_LIB"):
            continue  # an explicitly chosen oracle build (the mutation tests' broken copies)
        mod = _module_from_file(name, os.path.join(ROOT, *rel))
        if mod.up_to_date():
            continue
        if on_gpu_host:
            pytest.exit(f"{mod.LIB_PATH} is missing or older than its sources: build it first "
                        "(python __graft_entry__.py)", returncode=3)
        mod.build()


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
