"""The C ABI's host code under AddressSanitizer (no GPU).

libmoe.so is rebuilt with AddressSanitizer on its host code only
(build.py, host_asan_dir) and driven by asan_abi_driver.py in a child process
with the ASan runtime preloaded: argument checks of every entry point,
workspace sizing for many problems and moe_plan over host count arrays must
make no invalid host memory access. A caller's counts buffer one entry short
must be reported, which shows that the instrumentation is live.
"""

import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "asan_abi_driver.py")


def _asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not available")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the ASan runtime is not available")
    spec = importlib.util.spec_from_file_location(
        "_moe_build_asan", os.path.join(ROOT, "sparse_mixture_experts_route_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = mod.build(host_asan_dir=str(tmp_path_factory.mktemp("asan")))
    return lib, rt


def _run(asan_lib, *args):
    lib, rt = asan_lib
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    return subprocess.run([sys.executable, DRIVER, lib, *args], env=env, capture_output=True, text=True,
                          timeout=600)


def test_host_paths_make_no_invalid_access(asan_lib):
    r = _run(asan_lib)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr[-4000:]


def test_asan_reports_a_short_counts_buffer(asan_lib):
    r = _run(asan_lib, "--short-counts")
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-4000:]
