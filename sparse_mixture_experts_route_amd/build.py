"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libmoe.so")

SOURCES = ["route.hip", "permute.hip", "grouped_gemm.hip", "combine.hip", "grouped_gemm_bwd.hip", "backward.hip",
           "small_layer.hip", "moe_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns about the device-only target feature; that line is noise
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


# AddressSanitizer on the host code only (argument checks, workspace layout,
# launch planning); the device code is built as usual
HOST_ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, jobs: int = 8, host_asan_dir: str = "") -> str:
    """Compile every source for gfx950 and link libmoe.so next to this file. Always rebuilds.

    With host_asan_dir, build a copy whose host code carries AddressSanitizer
    instead, as host_asan_dir/libmoe_asan.so (a process loading it needs the
    ASan runtime preloaded); libmoe.so is left as it is."""
    cc = hipcc()
    bdir = host_asan_dir or BUILD_DIR
    out = os.path.join(bdir, "libmoe_asan.so") if host_asan_dir else LIB_PATH
    extra = HOST_ASAN_FLAGS if host_asan_dir else []
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *compile_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libsan"] if host_asan_dir else []
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *link_extra,
          "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
