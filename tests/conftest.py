import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_built():
    # Build only what is missing: the GPU runs use the in-tree libraries as built.
    from oracle import build as oracle_build
    if not os.path.exists(oracle_build.LIB):
        oracle_build.build()


_ensure_built()


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


def _ensure_hip_built():
    from exact_top_selection_stride_amd import build as hip_build
    if not os.path.exists(hip_build.LIB):
        hip_build.build()
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "mfma_probe_build", os.path.join(ROOT, "tests", "native", "build.py"))
    probe_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(probe_build)
    if not os.path.exists(probe_build.LIB):
        probe_build.build()


_ensure_hip_built()
