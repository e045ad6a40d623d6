"""Seeded random layer shapes on the GPU against the oracle.

Ragged groups, empty experts, E not a multiple of 8 (the router's FMA path),
k = E, tiny T, and every bf16 block tile, with and without a capped
persistent grid and forced splitting of leftover tiles: the scheduling paths
of the grouped GEMM (whole tiles, split tiles and their fixup, waves that
skip padding rows, the next tile's first stage issued during the epilogue)
all meet the same outputs.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, announce, check_routing_e2e, check_routing_exact, f64, needs_gpu, rel_err
from harness import host_array, make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]

TILES = ["auto", "256x256w8", "128x128", "256x128", "256x256", "256x256w8k32", "128x128k32"]
BASES = ["mixtral_coarse", "fine_grained", "skewed", "large_sparse"]


def make_cases(n=24, seed=2024, experts=(1, 3, 8, 12, 16, 40, 64)):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice(experts))
        k = int(rng.integers(1, min(E, 8) + 1)) if i % 7 else E if E <= 16 else 8
        cases.append(dict(
            base=BASES[i % len(BASES)],
            T=int(rng.choice([1, 7, 64, 333, 1000, 1999])),
            d_model=64 * int(rng.integers(1, 9)),
            d_expert=64 * int(rng.integers(1, 13)),
            E=E, k=k,
            dtype="f32" if i % 11 == 5 else "bf16",
            tile=TILES[int(rng.integers(0, len(TILES)))],
            blocks=[None, 8, 24, 64][int(rng.integers(0, 4))],
            split0=bool(rng.integers(0, 2)),
            seed=int(rng.integers(0, 1000)),
        ))
    return cases


# the first set, then wide expert counts: every padded router width (64,
# 128, 192, 256 columns), including 129 .. 192 experts
CASES = make_cases() + make_cases(n=8, seed=2025, experts=(72, 128, 136, 160, 192, 200, 256))


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_random_shape(moe, case):
    cfg = scaled_config(case["base"], T=case["T"], d_model=case["d_model"], E=case["E"], k=case["k"],
                        d_expert=case["d_expert"], dtype=case["dtype"], suffix="rand")
    announce(f"random {case}")
    env = {}
    if case["tile"] != "auto":
        env["MOE_GEMM_TILE"] = case["tile"]
    if case["blocks"]:
        env["MOE_GEMM_MAX_BLOCKS"] = str(case["blocks"])
    if case["split0"]:
        env["MOE_GEMM_SPLIT_MIN_STEPS"] = "0"
    inp = make_inputs(cfg, seed=case["seed"], device="cuda")
    os.environ.update(env)
    try:
        layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
        st = layer.stages(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
        y = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"]).clone()
        torch.cuda.synchronize()
    finally:
        for key in env:
            del os.environ[key]
    assert torch.equal(y, st["y"]), "moe_forward and the stage calls must agree bitwise"
    h = {key: host_array(v) for key, v in inp.items()}
    ref = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    logits, idx, _ = check_routing_exact(cfg, st)
    x64, wr64 = oracle.decode(h["x"], cfg.dtype), oracle.decode(h["w_router"], cfg.dtype)
    keep = check_routing_e2e(cfg, logits, idx, f64(st["gate"]), x64, wr64, h["router_bias"], ref)
    if keep.any():
        err = rel_err(f64(y)[keep], ref["y"][keep])
        assert err <= (TOL_F32 if cfg.dtype == "f32" else TOL_BF16), err
