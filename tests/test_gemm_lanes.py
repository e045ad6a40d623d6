"""Host replay of the grouped GEMM's lane address arithmetic (no GPU).

gemm_lanes_check.cpp includes the kernel's own lane arithmetic
(csrc/gemm_lanes.h) and walks every operand load and output store of the
tiles of one expert group, for every block-tile shape the kernel has, with
widths that are not multiples of the tile width: every access must stay
inside its operand (or be sent past the buffer range and read zero), and
every element a tile needs must come from exactly its own address.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_route_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "gemm_lanes_check.cpp")

TILES = [(256, 256, 64, 8), (256, 256, 32, 8), (256, 256, 64, 4), (256, 256, 32, 4), (256, 128, 32, 4),
         (128, 128, 64, 4), (128, 128, 32, 4), (32, 256, 64, 4)]
# (K, N, rows of the group, rows of the gathered operand)
SHAPES = [(128, 192, 300, 70), (192, 320, 37, 0), (64, 64, 1, 5), (256, 2048 + 64, 513, 0),
          (128, 448, 256, 3), (64, 128, 255, 0)]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("lanes") / "gemm_lanes_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-I", CSRC, SRC, "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("tile", TILES, ids=lambda t: "x".join(map(str, t)))
def test_loads_and_stores_stay_inside(checker, tile):
    for K, N, rows, a_rows in SHAPES:
        if K % tile[2]:
            continue
        r = subprocess.run([checker, *map(str, tile), str(K), str(N), str(rows), str(a_rows)],
                           capture_output=True, text=True)
        assert r.returncode == 0 and r.stdout.startswith("ok"), (tile, K, N, rows, r.stdout)


def test_checker_catches_a_load_past_the_slab(checker, tmp_path):
    """The replay flags the access pattern the tiles had when the last n-tile
    started at a multiple of the tile width: lanes past column N on the
    slab's last k row read past its end under a vector-offset-only range check."""
    src = open(SRC).read().replace("const int n0 = tile_n0(nt, n_tiles, N, BN);\n    if (n0",
                                   "const int n0 = nt * BN;\n    if (0 && n0")
    assert src != open(SRC).read()
    planted = tmp_path / "planted.cpp"
    planted.write_text(src)
    exe = str(tmp_path / "planted")
    cxx = shutil.which("g++") or shutil.which("c++")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", CSRC, str(planted), "-o", exe], check=True)
    r = subprocess.run([exe, "256", "256", "64", "8", "128", "320", "300", "0"], capture_output=True, text=True)
    assert r.returncode == 1 and r.stdout.startswith("FAIL B"), r.stdout
