"""moe_grouped_ffn on the GPU against the oracle's per-expert FFN on the same
permuted rows and group offsets (ragged, with empty groups and tile tails)."""

import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, announce, f64, needs_gpu, rel_err
from harness import host_array, make_dense, make_group_offsets

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_ffn(moe, R, d, de, E, dtype, x_perm, offsets, W1, W2):
    # the problem's T*k must cover the rows; use k = 1, T = R
    p = moe.make_problem(R, d, E, 1, de, dtype)
    y = torch.full((R, d), float("nan"), dtype=x_perm.dtype, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device="cuda")
    moe.moe_grouped_ffn(p, x_perm, offsets, W1, W2, y, ws)
    torch.cuda.synchronize()
    return y


def oracle_ffn(dtype, x_perm, offsets, W1, W2):
    xp = oracle.decode(host_array(x_perm), dtype)
    w1, w2 = host_array(W1), host_array(W2)
    return oracle.grouped_ffn(xp, host_array(offsets), lambda e: oracle.decode(w1[e], dtype),
                              lambda e: oracle.decode(w2[e], dtype))


CASES = [
    # R, d, de, E, dtype, empty groups
    (1, 64, 64, 1, "bf16", ()),
    (100, 128, 256, 8, "f32", ()),
    (777, 256, 192, 5, "f32", (2,)),
    (300, 128, 256, 8, "bf16", ()),
    (1000, 256, 512, 8, "bf16", (3, 4)),
    (2500, 512, 384, 16, "bf16", (0, 15)),
    (4096, 1024, 1024, 4, "bf16", ()),
    (1537, 192, 320, 64, "bf16", tuple(range(30, 60))),
]


@pytest.mark.parametrize("R,d,de,E,dtype,empty", CASES)
def test_grouped_ffn_against_oracle(moe, R, d, de, E, dtype, empty):
    announce(f"ffn R={R} d={d} de={de} E={E} {dtype} empty={len(empty)}")
    x_perm = make_dense((R, d), 1.0, seed=6, tag=1, device="cuda", dtype=dtype)
    W1 = make_dense((E, d, de), d ** -0.5, seed=6, tag=2, device="cuda", dtype=dtype)
    W2 = make_dense((E, de, d), de ** -0.5, seed=6, tag=3, device="cuda", dtype=dtype)
    off = make_group_offsets(E, R, seed=6, empty=empty)
    y = run_ffn(moe, R, d, de, E, dtype, x_perm, off.cuda(), W1, W2)
    ref = oracle_ffn(dtype, x_perm, off, W1, W2)
    err = rel_err(f64(y), ref)
    print(f"ffn R={R} d={d} de={de} E={E} {dtype}: rel err {err:.3e}")
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)


@pytest.mark.parametrize("tile", ["256x256", "256x256k32", "256x128", "128x128", "128x128k32", "256x256w8", "256x256w8k32",
                                  "32x256"])
def test_every_tile_shape(moe, tile):
    """Each bf16 block tile the launcher can choose, on ragged groups with
    empty experts and rows that are not a multiple of any tile."""
    R, d, de, E = 1299, 512, 768, 6
    announce(f"ffn tile {tile}")
    x_perm = make_dense((R, d), 1.0, seed=7, tag=1, device="cuda")
    W1 = make_dense((E, d, de), d ** -0.5, seed=7, tag=2, device="cuda")
    W2 = make_dense((E, de, d), de ** -0.5, seed=7, tag=3, device="cuda")
    off = make_group_offsets(E, R, seed=7, empty=(1,))
    os.environ["MOE_GEMM_TILE"] = tile
    try:
        y = run_ffn(moe, R, d, de, E, "bf16", x_perm, off.cuda(), W1, W2)
    finally:
        del os.environ["MOE_GEMM_TILE"]
    ref = oracle_ffn("bf16", x_perm, off, W1, W2)
    assert rel_err(f64(y), ref) <= TOL_BF16


@pytest.mark.parametrize("blocks", [24, 64])
@pytest.mark.parametrize("tile", ["256x256w8", "128x128", "256x128", "32x256"])
@pytest.mark.parametrize("R,d,de,E", [(20000, 128, 64, 3), (9000, 512, 64, 2), (6000, 256, 192, 7)])
def test_split_leftover_tiles(moe, tile, R, d, de, E, blocks):
    """A capped persistent grid gives several rounds of tiles and a small
    leftover, whose K steps are split over the blocks: tiles summed from
    several blocks' partial sums, and (K of one or two steps) shares that are a
    whole tile, stored by the block itself and skipped by the fixup."""
    announce(f"ffn split tiles {tile} blocks={blocks} R={R} d={d} de={de} E={E}")
    x_perm = make_dense((R, d), 1.0, seed=9, tag=1, device="cuda")
    W1 = make_dense((E, d, de), d ** -0.5, seed=9, tag=2, device="cuda")
    W2 = make_dense((E, de, d), de ** -0.5, seed=9, tag=3, device="cuda")
    off = make_group_offsets(E, R, seed=9)
    env = {"MOE_GEMM_TILE": tile, "MOE_GEMM_MAX_BLOCKS": str(blocks), "MOE_GEMM_SPLIT_MIN_STEPS": "0"}
    os.environ.update(env)
    try:
        y = run_ffn(moe, R, d, de, E, "bf16", x_perm, off.cuda(), W1, W2)
    finally:
        for k in env:
            del os.environ[k]
    ref = oracle_ffn("bf16", x_perm, off, W1, W2)
    assert rel_err(f64(y), ref) <= TOL_BF16


def test_rows_past_offsets_end_untouched(moe):
    """Rows at or beyond offsets[E] belong to no expert and keep their contents."""
    R, d, de, E = 500, 128, 128, 4
    announce("ffn rows past end")
    x_perm = make_dense((R, d), 1.0, seed=8, tag=1, device="cuda")
    W1 = make_dense((E, d, de), d ** -0.5, seed=8, tag=2, device="cuda")
    W2 = make_dense((E, de, d), de ** -0.5, seed=8, tag=3, device="cuda")
    off = make_group_offsets(E, 420, seed=8)
    y = run_ffn(moe, R, d, de, E, "bf16", x_perm, off.cuda(), W1, W2)
    assert torch.isnan(y[420:].float()).all()
    ref = oracle_ffn("bf16", x_perm[:420], off, W1, W2)
    assert rel_err(f64(y[:420]), ref) <= TOL_BF16


@pytest.mark.parametrize("tile,split0", [("auto", False), ("256x256w8", True), ("128x128", False),
                                         ("256x128", True), ("256x256w8k32", False), ("32x256", True),
                                         ("32x256", False)])
def test_gather_path_matches_permuted_copy(moe, tile, split0):
    """moe_permute_index + moe_grouped_ffn_gather (the first GEMM reads x[perm[r]])
    give the same index arrays and the same y_perm, bit for bit, as moe_permute
    + moe_grouped_ffn on the copied x_perm."""
    from harness import make_inputs, scaled_config
    cfg = scaled_config("skewed", T=1500, d_model=256, E=16, k=4, d_expert=320)
    announce(f"ffn gather {tile} split0={split0}")
    inp = make_inputs(cfg, seed=3, device="cuda")
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    p = layer.problem
    env = {"MOE_GEMM_MAX_BLOCKS": "24"}
    if tile != "auto":
        env["MOE_GEMM_TILE"] = tile
    if split0:
        env["MOE_GEMM_SPLIT_MIN_STEPS"] = "0"
    os.environ.update(env)
    try:
        st = layer.stages(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
        R = cfg.T * cfg.k
        dev = "cuda"
        counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(R, dtype=torch.int32, device=dev)
        inv = torch.empty(R, dtype=torch.int32, device=dev)
        ws_p = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_PERMUTE), dtype=torch.uint8, device=dev)
        ws_f = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device=dev)
        y_perm = torch.full((R, cfg.d_model), float("nan"), dtype=inp["x"].dtype, device=dev)
        moe.moe_permute_index(p, st["idx"], counts, offsets, perm, inv, ws_p)
        moe.moe_grouped_ffn_gather(p, inp["x"], perm, offsets, inp["W1"], inp["W2"], y_perm, ws_f)
        torch.cuda.synchronize()
    finally:
        for key in env:
            del os.environ[key]
    for name, t in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv)):
        assert torch.equal(t, st[name]), name
    assert torch.equal(y_perm, st["y_perm"])


@pytest.mark.parametrize("blocks,split0", [(24, True), (64, False), (256, False)])
def test_raster_groups_do_not_change_results(moe, blocks, split0):
    """The order in which an expert's tiles are dealt to blocks (m-tiles in
    raster groups of MOE_GEMM_GROUP_M, or one group) changes no sum: the
    outputs are equal bit for bit, with experts of many m-tiles, split
    leftover tiles and the row-gathering first GEMM."""
    R, d, de, E = 9000, 256, 320, 3
    announce(f"ffn raster groups blocks={blocks} split0={split0}")
    x = make_dense((R, d), 1.0, seed=12, tag=1, device="cuda")
    W1 = make_dense((E, d, de), d ** -0.5, seed=12, tag=2, device="cuda")
    W2 = make_dense((E, de, d), de ** -0.5, seed=12, tag=3, device="cuda")
    off = make_group_offsets(E, R, seed=12).cuda()
    perm = torch.arange(R, dtype=torch.int32, device="cuda")
    p = moe.make_problem(R, d, E, 1, de, "bf16")
    out = {}
    for gm in ("0", "1", "3", "8"):
        env = {"MOE_GEMM_MAX_BLOCKS": str(blocks), "MOE_GEMM_GROUP_M": gm}
        if split0:
            env["MOE_GEMM_SPLIT_MIN_STEPS"] = "0"
        os.environ.update(env)
        try:
            y = run_ffn(moe, R, d, de, E, "bf16", x, off, W1, W2)
            ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device="cuda")
            yg = torch.full_like(y, float("nan"))
            moe.moe_grouped_ffn_gather(p, x, perm, off, W1, W2, yg, ws)
            torch.cuda.synchronize()
        finally:
            for k in env:
                del os.environ[k]
        out[gm] = (y, yg)
    for gm in ("1", "3", "8"):
        assert torch.equal(out[gm][0], out["0"][0]), gm
        assert torch.equal(out[gm][1], out["0"][1]), gm
    ref = oracle_ffn("bf16", x, off.cpu(), W1, W2)
    assert rel_err(f64(out["8"][0]), ref) <= TOL_BF16



@pytest.mark.parametrize("blocks", [64, 256])
def test_fixup_rounds_do_not_change_results(moe, blocks):
    """A fixup block may complete several split tiles in turn
    (MOE_FIXUP_ROUNDS): each tile's partial sums are added in K order whichever
    block takes it, so the outputs are equal bit for bit."""
    R, d, de, E = 20000, 256, 192, 5
    announce(f"ffn fixup rounds blocks={blocks}")
    x = make_dense((R, d), 1.0, seed=14, tag=1, device="cuda")
    W1 = make_dense((E, d, de), d ** -0.5, seed=14, tag=2, device="cuda")
    W2 = make_dense((E, de, d), de ** -0.5, seed=14, tag=3, device="cuda")
    off = make_group_offsets(E, R, seed=14).cuda()
    out = {}
    for rounds in ("1", "2", "4"):
        env = {"MOE_GEMM_MAX_BLOCKS": str(blocks), "MOE_GEMM_SPLIT_MIN_STEPS": "0", "MOE_FIXUP_ROUNDS": rounds,
               "MOE_GEMM_TILE": "256x256w8"}
        os.environ.update(env)
        try:
            out[rounds] = run_ffn(moe, R, d, de, E, "bf16", x, off, W1, W2)
        finally:
            for k in env:
                del os.environ[k]
    assert torch.equal(out["2"], out["1"]) and torch.equal(out["4"], out["1"])
    ref = oracle_ffn("bf16", x, off.cpu(), W1, W2)
    assert rel_err(f64(out["4"]), ref) <= TOL_BF16


@pytest.mark.parametrize("blocks", [24, 64, 256])
def test_split_completion_in_launch_matches_fixup(moe, blocks):
    """The 32-row weight-streaming tile can complete its split tiles inside
    the GEMM launch (forced here for both GEMMs): the last block to store a
    tile's partial sums adds all of its slots in K order. Outputs equal those
    of the fixup launch bit for bit, for both FFN entry points and on three
    calls in a row (each launch leaves its tile counters at zero for the next)."""
    R, d, de, E = 3001, 512, 768, 7
    announce(f"ffn split completion in launch blocks={blocks}")
    x = make_dense((R, d), 1.0, seed=15, tag=1, device="cuda")
    W1 = make_dense((E, d, de), d ** -0.5, seed=15, tag=2, device="cuda")
    W2 = make_dense((E, de, d), de ** -0.5, seed=15, tag=3, device="cuda")
    off = make_group_offsets(E, R, seed=15, empty=(2,)).cuda()
    perm = torch.randperm(R, generator=torch.Generator().manual_seed(15)).to(torch.int32).cuda()
    p = moe.make_problem(R, d, E, 1, de, "bf16")

    def both():
        y = run_ffn(moe, R, d, de, E, "bf16", x, off, W1, W2)
        ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device="cuda")
        yg = torch.full_like(y, float("nan"))
        moe.moe_grouped_ffn_gather(p, x, perm, off, W1, W2, yg, ws)
        torch.cuda.synchronize()
        return y, yg

    env = {"MOE_GEMM_TILE": "32x256", "MOE_GEMM_MAX_BLOCKS": str(blocks), "MOE_GEMM_SPLIT_MIN_STEPS": "0"}
    os.environ.update(env)
    try:
        os.environ["MOE_GEMM_SPLIT_FIXUP"] = "1"
        ref = both()
        del os.environ["MOE_GEMM_SPLIT_FIXUP"]
        os.environ["MOE_GEMM_SPLIT_INLAUNCH"] = "1"
        runs = [both() for _ in range(3)]
    finally:
        os.environ.pop("MOE_GEMM_SPLIT_FIXUP", None)
        os.environ.pop("MOE_GEMM_SPLIT_INLAUNCH", None)
        for k in env:
            del os.environ[k]
    for i, (y, yg) in enumerate(runs):
        assert torch.equal(y, ref[0]), i
        assert torch.equal(yg, ref[1]), i
    xr = oracle.decode(host_array(x), "bf16")[host_array(perm).astype(np.int64)]
    w1, w2 = host_array(W1), host_array(W2)
    want = oracle.grouped_ffn(xr, host_array(off), lambda e: oracle.decode(w1[e], "bf16"),
                              lambda e: oracle.decode(w2[e], "bf16"))
    assert rel_err(f64(runs[2][1]), want) <= TOL_BF16
