"""Decode-sized batches (a few tokens, k = 1 or the workloads' k) at the
workloads' full layer widths, against the oracle on every token.

These take the launch configuration the library picks for small T: the router
split over d_model (float32 partial logits, summed in a fixed order by a
second launch) and the 32-row GEMM tile with a block per CU slot, whose one
partly filled round of weight slabs is split over all blocks by K steps.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, announce, check_routing_e2e, check_routing_exact, f64, needs_gpu, rel_err
from harness import host_array, make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [
    # workload, T, k (None: the workload's)
    ("mixtral_coarse", 1, None),
    ("mixtral_coarse", 7, None),
    ("mixtral_coarse", 64, None),
    ("mixtral_coarse", 160, None),   # 40 rows per expert: the largest batch on the 32-row tile
    ("mixtral_coarse", 32, 1),
    ("fine_grained", 8, None),
    ("fine_grained", 64, None),
    ("fine_grained", 16, 1),
    ("skewed", 33, None),
    ("large_sparse", 8, None),
]


@pytest.mark.parametrize("name,T,k", CASES)
def test_forward_decode_sized(moe, name, T, k):
    cfg = scaled_config(name, T=T, k=k, suffix="decode")
    announce(f"forward decode {cfg.name} T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k} de={cfg.d_expert}")
    inp = make_inputs(cfg, seed=5, device="cuda")
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    st = layer.stages(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    y = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(y, st["y"]), "moe_forward and the four stage calls must agree bitwise"

    W1, W2 = inp["W1"], inp["W2"]
    ref = oracle.forward_tokens(host_array(inp["x"]), host_array(inp["w_router"]), host_array(inp["router_bias"]),
                                lambda e: host_array(W1[e]), lambda e: host_array(W2[e]), cfg.k, cfg.dtype)
    logits, idx, _ = check_routing_exact(cfg, st)
    x64 = oracle.decode(host_array(inp["x"]), cfg.dtype)
    wr64 = oracle.decode(host_array(inp["w_router"]), cfg.dtype)
    keep = check_routing_e2e(cfg, logits, idx, f64(st["gate"]), x64, wr64, host_array(inp["router_bias"]), ref)
    err = rel_err(f64(y)[keep], ref["y"][keep])
    print(f"{cfg.name} T={T} k={cfg.k}: y rel err {err:.3e}, near-ties excluded {int((~keep).sum())}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("mode", ["default", "inlaunch"])
@pytest.mark.parametrize("name,T", [("mixtral_coarse", 1), ("mixtral_coarse", 32), ("fine_grained", 8),
                                    ("skewed", 33)])
def test_decode_split_completion_in_launch(moe, name, T, mode):
    """moe_forward at decode sizes with split tiles completed inside the GEMM
    launches (the library's choice per GEMM, or forced for both): y equals,
    bit for bit, the layer run with fixup launches, on three calls in a row."""
    cfg = scaled_config(name, T=T, suffix="decode")
    announce(f"forward decode in-launch completion {cfg.name} T={cfg.T}")
    inp = make_inputs(cfg, seed=6, device="cuda")
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    args = (inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    os.environ["MOE_GEMM_SPLIT_FIXUP"] = "1"
    try:
        ref = layer(*args).clone()
    finally:
        del os.environ["MOE_GEMM_SPLIT_FIXUP"]
    if mode == "inlaunch":
        os.environ["MOE_GEMM_SPLIT_INLAUNCH"] = "1"
    try:
        ys = [layer(*args).clone() for _ in range(3)]
        torch.cuda.synchronize()
    finally:
        os.environ.pop("MOE_GEMM_SPLIT_INLAUNCH", None)
    for i, y in enumerate(ys):
        assert torch.equal(y, ref), i
