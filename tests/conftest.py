import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload run")


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()


def _ensure_built():
    """Build libmoe.so only when nothing is built yet (a build is a separate step)."""
    lib = os.path.join(ROOT, "sparse_mixture_experts_route_amd", "libmoe.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "sparse_mixture_experts_route_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return lib


@pytest.fixture(scope="session")
def libmoe_path():
    return _ensure_built()


@pytest.fixture(scope="session")
def moe(libmoe_path):
    import sparse_mixture_experts_route_amd as m
    return m
