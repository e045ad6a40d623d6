"""moe_route on the GPU against the CPU oracle's router (Linear + softmax + top-k)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import U32, announce, check_topk_valid, f64, i64, logit_bound, needs_gpu
from harness import CONFIGS, host_array, make_exact_router_inputs, make_inputs, scaled_config
from harness.configs import CONFIG_ORDER

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_route(moe, cfg, x, wr, bias, via="moe_route"):
    """Route through moe_route, or through moe_route_ws (which splits the
    contraction over d_model when the tokens alone do not fill the GPU)."""
    p = moe.make_problem(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, cfg.dtype)
    dev = x.device
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    if via == "moe_route":
        call = lambda lg, i, g: moe.moe_route(p, x, wr, bias, lg, i, g)  # noqa: E731
    else:
        ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_ROUTE), dtype=torch.uint8, device=dev)
        call = lambda lg, i, g: moe.moe_route_ws(p, x, wr, bias, lg, i, g, ws)  # noqa: E731
    call(logits, idx, gate)
    # the same routing without exporting logits
    idx2 = torch.empty_like(idx)
    gate2 = torch.empty_like(gate)
    call(None, idx2, gate2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(gate, gate2)
    return f64(logits).astype(np.float32), i64(idx), f64(gate)


@pytest.mark.parametrize("via", ["moe_route", "moe_route_ws"])
@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_route_full_size_against_oracle(moe, name, via):
    """Every workload at full size: logits within the float32 rounding bound,
    selected sets equal outside near-ties, gates within the bound implied by
    the logit difference, and idx exactly the top-k of the GPU's own logits."""
    cfg = CONFIGS[name]
    announce(f"route full {name} via {via} T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k}")
    inp = make_inputs(cfg, seed=0, device="cuda", weights=False)
    logits, idx, gate = run_route(moe, cfg, inp["x"], inp["w_router"], inp["router_bias"], via)
    xh, wh, bh = host_array(inp["x"]), host_array(inp["w_router"]), host_array(inp["router_bias"])
    x64, w64 = oracle.decode(xh, cfg.dtype), oracle.decode(wh, cfg.dtype)
    ref = oracle.route(x64, w64, bh, cfg.k)

    dl = np.abs(logits.astype(np.float64) - ref["logits"].astype(np.float64))
    bound = logit_bound(x64, w64, bh, ref["logits"])
    assert np.all(dl <= bound), f"logit error {dl.max():.3e} above bound"

    check_topk_valid(idx, logits)
    tie = ref["near_tie"]
    same = np.array([set(idx[t]) == set(ref["idx"][t]) for t in range(cfg.T)])
    bad = np.nonzero(~same & ~tie)[0]
    assert bad.size == 0, f"{bad.size} tokens route differently outside near-ties, e.g. {bad[:5]}"
    print(f"{name}: max|dlogit|={dl.max():.3e} near_ties={int(tie.sum())} "
          f"differing(near-tie)={int((~same).sum())}")

    ok = same & ~tie
    # the oracle's gate of each expert the GPU selected (same set on these tokens)
    rg = np.ones_like(gate)
    for t in np.nonzero(ok)[0]:
        by_e = dict(zip(ref["idx"][t].tolist(), ref["gate"][t].tolist()))
        rg[t] = [by_e[int(e)] for e in idx[t]]
    rel = np.abs(gate - rg) / rg
    tol = 2 * dl.max(axis=1, keepdims=True) + 32 * U32
    assert np.all(rel[ok] <= np.broadcast_to(tol, rel.shape)[ok]), f"gate error {rel[ok].max():.3e}"


@pytest.mark.parametrize("via", ["moe_route", "moe_route_ws"])
@pytest.mark.parametrize("tie_group", [1, 3])
@pytest.mark.parametrize("name,T,d,bias", [
    ("tiny_fp32", 200, 128, False),
    ("mixtral_coarse", 333, 2048, False),
    ("fine_grained", 517, 2048, True),
    ("large_sparse", 130, 7168, True),
    # decode-sized batches: moe_route_ws splits these over d_model
    ("mixtral_coarse", 1, 2048, False),
    ("large_sparse", 8, 7168, True),
    ("fine_grained", 64, 1024, True),
])
def test_route_bit_exact_on_exact_logits(moe, name, T, d, bias, tie_group, via):
    """Inputs whose float32 logits are exact in any summation order: logits and
    indices must be bit-exact, gates within the float32 softmax rounding bound.
    With tie_group=3 experts tie in threes, so the lowest-index rule decides
    the k-th place of every token."""
    cfg = scaled_config(name, T=T, d_model=d)
    announce(f"route exact {cfg.name} via {via} T={T} d={d} E={cfg.E} k={cfg.k} bias={bias} ties={tie_group}")
    inp = make_exact_router_inputs(cfg, seed=1, device="cuda", bias=bias, tie_group=tie_group)
    logits, idx, gate = run_route(moe, cfg, inp["x"], inp["w_router"], inp["router_bias"], via)
    bh = host_array(inp["router_bias"])
    ref = oracle.route(oracle.decode(host_array(inp["x"]), cfg.dtype),
                       oracle.decode(host_array(inp["w_router"]), cfg.dtype), bh, cfg.k)
    assert np.array_equal(logits, ref["logits"])
    assert np.array_equal(idx, ref["idx"])
    np.testing.assert_allclose(gate, ref["gate"], rtol=32 * U32, atol=0)
    # ties at the selection boundary really occurred
    s = -np.sort(-ref["logits"], axis=1)
    n_ties = int(np.sum(s[:, cfg.k - 1] == s[:, cfg.k])) if cfg.k < cfg.E else 0
    print(f"{cfg.name}: {n_ties} tokens with a tie at the k-th place")
    if tie_group > 1 and cfg.k < cfg.E:
        assert n_ties > cfg.T // 4


@pytest.mark.parametrize("E,k", [(8, 8), (64, 64), (256, 3), (1, 1), (256, 256)])
def test_route_extreme_k(moe, E, k):
    cfg = scaled_config("fine_grained", T=70, d_model=128, E=E, k=k)
    announce(f"route extreme E={E} k={k}")
    inp = make_exact_router_inputs(cfg, seed=2, device="cuda", bias=True)
    logits, idx, gate = run_route(moe, cfg, inp["x"], inp["w_router"], inp["router_bias"])
    bh = host_array(inp["router_bias"])
    ref = oracle.route(oracle.decode(host_array(inp["x"]), cfg.dtype),
                       oracle.decode(host_array(inp["w_router"]), cfg.dtype), bh, cfg.k)
    assert np.array_equal(idx, ref["idx"])
    np.testing.assert_allclose(gate, ref["gate"], rtol=32 * U32 + E * U32, atol=0)


def test_route_zero_router_ties_to_lowest_index(moe):
    cfg = scaled_config("large_sparse", T=33, d_model=256)
    announce("route zero router")
    inp = make_inputs(cfg, seed=0, device="cuda", router_zero=True, weights=False)
    logits, idx, gate = run_route(moe, cfg, inp["x"], inp["w_router"], None)
    assert np.all(logits == 0)
    assert np.array_equal(idx, np.tile(np.arange(cfg.k), (cfg.T, 1)))
    assert np.all(gate == np.float32(1.0 / cfg.E))


@pytest.mark.parametrize("rt", ["32", "64"])
@pytest.mark.parametrize("name,T,d,E,k", [
    ("fine_grained", 517, 2048, 64, 6),
    ("skewed", 1000, 1024, 128, 8),
    ("large_sparse", 95, 1024, 256, 8),
    ("fine_grained", 77, 512, 192, 12),
    ("fine_grained", 300, 1024, 136, 4),
    ("skewed", 129, 768, 160, 2),
])
def test_route_block_sizes_bit_exact(moe, rt, name, T, d, E, k):
    """The matrix-core router's block of 32 or 64 tokens (MOE_ROUTE_RT): on
    inputs whose logits are exact, logits and indices equal the oracle's bit
    for bit, with ragged last blocks, every padded expert width (64 .. 256,
    also 192, whose w_router rows hold 24 LDS chunks) and k beyond the
    register top-k list."""
    import os
    cfg = scaled_config(name, T=T, d_model=d, E=E, k=k)
    announce(f"route block {rt} {name} T={T} d={d} E={E} k={k}")
    inp = make_exact_router_inputs(cfg, seed=4, device="cuda", bias=True, tie_group=3)
    os.environ["MOE_ROUTE_RT"] = rt
    try:
        for via in ("moe_route", "moe_route_ws"):
            logits, idx, gate = run_route(moe, cfg, inp["x"], inp["w_router"], inp["router_bias"], via)
            ref = oracle.route(oracle.decode(host_array(inp["x"]), cfg.dtype),
                               oracle.decode(host_array(inp["w_router"]), cfg.dtype),
                               host_array(inp["router_bias"]), cfg.k)
            assert np.array_equal(logits, ref["logits"]), via
            assert np.array_equal(idx, ref["idx"]), via
            np.testing.assert_allclose(gate, ref["gate"], rtol=32 * U32, atol=0)
    finally:
        del os.environ["MOE_ROUTE_RT"]
