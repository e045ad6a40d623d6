"""Degenerate and edge cases of the layer, determinism, and stream handling."""

import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, announce, f64, i64, needs_gpu, rel_err
from harness import host_array, make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_and_compare(moe, cfg, inp, tol):
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    st = layer.stages(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    torch.cuda.synchronize()
    h = {k: host_array(v) for k, v in inp.items()}
    ref = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    keep = ~ref["near_tie"]
    err = rel_err(f64(st["y"])[keep], ref["y"][keep])
    assert err <= tol, err
    return st, ref


def test_zero_router_everything_ties(moe):
    cfg = scaled_config("fine_grained", T=300, d_model=128, d_expert=128)
    announce("special zero router")
    inp = make_inputs(cfg, seed=0, device="cuda", router_zero=True)
    st, ref = run_and_compare(moe, cfg, inp, TOL_BF16)
    assert np.array_equal(i64(st["idx"]), np.tile(np.arange(cfg.k), (cfg.T, 1)))
    assert np.all(f64(st["gate"]) == np.float32(1 / cfg.E))
    assert np.array_equal(i64(st["counts"]), ref["counts"])  # all rows in experts 0..k-1


def test_k_equals_E_identical_experts_is_dense(moe):
    cfg = scaled_config("mixtral_coarse", T=200, d_model=256, d_expert=512, E=4, k=4)
    announce("special k=E identical experts")
    inp = make_inputs(cfg, seed=1, device="cuda")
    inp["W1"][:] = inp["W1"][0:1].clone()
    inp["W2"][:] = inp["W2"][0:1].clone()
    st, ref = run_and_compare(moe, cfg, inp, TOL_BF16)
    assert np.array_equal(i64(st["counts"]), np.full(cfg.E, cfg.T))
    np.testing.assert_allclose(f64(st["gate"]).sum(axis=1), 1.0, rtol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_expert(moe, dtype):
    cfg = scaled_config("tiny_fp32", T=77, d_model=128, d_expert=256, E=1, k=1, dtype=dtype)
    announce(f"special E=1 {dtype}")
    inp = make_inputs(cfg, seed=2, device="cuda")
    st, _ = run_and_compare(moe, cfg, inp, TOL_BF16 if dtype == "bf16" else TOL_F32)
    assert np.all(f64(st["gate"]) == 1.0)


def test_forced_empty_groups(moe):
    cfg = scaled_config("skewed", T=700, d_model=256, d_expert=256)
    announce("special forced empty groups")
    inp = make_inputs(cfg, seed=3, device="cuda")
    inp["router_bias"] = torch.zeros(cfg.E, device="cuda")
    inp["router_bias"][10:40] = -1e4
    st, ref = run_and_compare(moe, cfg, inp, TOL_BF16)
    assert np.all(i64(st["counts"])[10:40] == 0)


@pytest.mark.parametrize("T", [1, 2, 77, 257])
def test_odd_token_counts(moe, T):
    cfg = scaled_config("large_sparse", T=T, d_model=256, d_expert=128)
    announce(f"special T={T}")
    inp = make_inputs(cfg, seed=4, device="cuda")
    run_and_compare(moe, cfg, inp, TOL_BF16)


def test_deterministic_and_stream_aware(moe):
    cfg = scaled_config("fine_grained", T=1000, d_model=512, d_expert=256)
    announce("special determinism/streams")
    inp = make_inputs(cfg, seed=5, device="cuda")
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    y1 = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"]).clone()
    y2 = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"]).clone()
    side = torch.cuda.Stream()  # default priority
    layer2 = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y3 = layer2(inp["x"], inp["w_router"], inp["W1"], inp["W2"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_one_hip_runtime_in_process(moe):
    """libmoe.so must share torch's HIP runtime (one libamdhip64 mapped)."""
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
    assert any(moe.lib_path() in line for line in maps.splitlines())


@pytest.mark.parametrize("T,k", [(1500, 16), (40, 256)])
def test_max_experts_large_k(moe, T, k):
    """256 experts (the limit) with k past the register fast paths: the
    router's general selection, the permute's selections in groups of 8,
    and the combine's loop over selections; whole layer and stages agree."""
    cfg = scaled_config("large_sparse", T=T, d_model=128, d_expert=64, E=256, k=k)
    announce(f"special E=256 k={k} T={T}")
    inp = make_inputs(cfg, seed=5, device="cuda")
    st, ref = run_and_compare(moe, cfg, inp, TOL_BF16)
    assert np.array_equal(i64(st["counts"]), ref["counts"])
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    y = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y, st["y"])
