"""moe_forward_train + moe_backward on the GPU against the backward oracle.

Oracle-sized versions of the workloads (and a decode-sized batch) are
compared element by element: dx, the router weight and bias gradients, the
expert weight gradients (including experts that receive no token) and the
router load statistics. bf16 results meet max|d|/max|ref| <= 1e-2; the
float32 statistics are tighter.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, announce, f64, needs_gpu, rel_err
from harness import host_array, make_dense, make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [
    # workload, overrides
    ("mixtral_coarse", dict(T=256, d_model=256, d_expert=512)),
    ("fine_grained", dict(T=320, d_model=256, d_expert=256)),
    ("skewed", dict(T=400, d_model=256, d_expert=192)),
    ("large_sparse", dict(T=96, d_model=512, E=64, d_expert=256)),
    ("mixtral_coarse", dict(T=8, d_model=512, d_expert=1024)),
    ("fine_grained", dict(T=64, d_model=256, d_expert=256, k=1)),
]


def run_train(moe, cfg, inp, dy):
    dev = inp["x"].device
    p = moe.make_problem(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_TRAIN), dtype=torch.uint8, device=dev)
    bf = torch.bfloat16
    y = torch.empty((cfg.T, cfg.d_model), dtype=bf, device=dev)
    out = {
        "dx": torch.full((cfg.T, cfg.d_model), float("nan"), dtype=bf, device=dev),
        "dw_router": torch.full((cfg.d_model, cfg.E), float("nan"), dtype=bf, device=dev),
        "dbias": torch.full((cfg.E,), float("nan"), dtype=torch.float32, device=dev),
        "dW1": torch.full((cfg.E, cfg.d_model, cfg.d_expert), float("nan"), dtype=bf, device=dev),
        "dW2": torch.full((cfg.E, cfg.d_expert, cfg.d_model), float("nan"), dtype=bf, device=dev),
        "load_frac": torch.full((cfg.E,), float("nan"), dtype=torch.float32, device=dev),
        "mean_prob": torch.full((cfg.E,), float("nan"), dtype=torch.float32, device=dev),
    }
    moe.moe_forward_train(p, inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"], y, ws)
    moe.moe_backward(p, inp["x"], inp["w_router"], inp["W1"], inp["W2"], dy, out["dx"], out["dw_router"],
                     out["dbias"], out["dW1"], out["dW2"], out["load_frac"], out["mean_prob"], ws)
    torch.cuda.synchronize()
    return y, out


@pytest.mark.parametrize("name,over", CASES)
def test_backward_against_oracle(moe, name, over):
    cfg = scaled_config(name, suffix="bwd", **over)
    announce(f"backward {cfg.name} T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k} de={cfg.d_expert}")
    inp = make_inputs(cfg, seed=2, device="cuda")
    dy = make_dense((cfg.T, cfg.d_model), 1.0, seed=2, tag=9, device="cuda")
    y, g = run_train(moe, cfg, inp, dy)
    # the forward result of the training call matches the layer (H is GELU of the rounded U)
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    y_inf = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    torch.cuda.synchronize()
    assert rel_err(f64(y), f64(y_inf)) <= 1e-2

    h = {kk: host_array(v) for kk, v in inp.items()}
    ref = oracle.backward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype,
                          host_array(dy))
    assert not ref["near_tie"].any(), "choose a seed without near-ties: the gradients depend on the selection"
    for key in ("dx", "dw_router", "dW1", "dW2"):
        err = rel_err(f64(g[key]), ref[key])
        print(f"{cfg.name} {key}: rel err {err:.3e}")
        assert err <= TOL_BF16, key
    # dbias is a float32 sum over tokens of router-logit gradients that come from
    # the bf16 expert outputs (through the softmax Jacobian, which cancels): the
    # bf16 bar applies, like the router weight gradient
    err = rel_err(f64(g["dbias"]), ref["dbias"])
    print(f"{cfg.name} dbias: rel err {err:.3e}")
    assert err <= TOL_BF16
    np.testing.assert_allclose(f64(g["load_frac"]), ref["load_frac"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(f64(g["mean_prob"]), ref["mean_prob"], rtol=1e-4, atol=1e-7)
    # experts without tokens get exactly zero weight gradients
    for e in np.nonzero(ref["counts"] == 0)[0]:
        assert torch.count_nonzero(g["dW1"][e]) == 0 and torch.count_nonzero(g["dW2"][e]) == 0


@pytest.mark.parametrize("blocks", [24, 64])
def test_backward_split_last_round(moe, blocks):
    """A capped persistent grid gives the row-grouped backward GEMMs several
    rounds of tiles and a small last round split over the blocks by K steps
    (float32 partial sums added by the fixup), and x^T dlogit split over
    token ranges: the gradients are those of the unsplit run."""
    import os
    cfg = scaled_config("skewed", T=1200, d_model=512, E=16, k=4, d_expert=256, suffix="bwd")
    announce(f"backward split blocks={blocks}")
    inp = make_inputs(cfg, seed=6, device="cuda")
    dy = make_dense((cfg.T, cfg.d_model), 1.0, seed=6, tag=9, device="cuda")
    env = {"MOE_GEMM_MAX_BLOCKS": str(blocks), "MOE_GEMM_SPLIT_MIN_STEPS": "0"}
    os.environ.update(env)
    try:
        _, g = run_train(moe, cfg, inp, dy)
    finally:
        for key in env:
            del os.environ[key]
    h = {kk: host_array(v) for kk, v in inp.items()}
    ref = oracle.backward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype,
                          host_array(dy))
    assert not ref["near_tie"].any()
    for key in ("dx", "dw_router", "dW1", "dW2"):
        err = rel_err(f64(g[key]), ref[key])
        print(f"split blocks={blocks} {key}: rel err {err:.3e}")
        assert err <= TOL_BF16, key


@pytest.mark.parametrize("blocks", [24, 64])
def test_backward_raster_groups_do_not_change_results(moe, blocks):
    """The row-grouped backward GEMMs and their split fixup deal an expert's
    tiles in raster groups of MOE_GEMM_GROUP_M m-tiles: every gradient equals
    the one-group run bit for bit."""
    import os
    cfg = scaled_config("skewed", T=12000, d_model=512, E=8, k=2, d_expert=256, suffix="bwdgm")
    announce(f"backward raster groups blocks={blocks}")
    inp = make_inputs(cfg, seed=8, device="cuda")
    dy = make_dense((cfg.T, cfg.d_model), 1.0, seed=8, tag=9, device="cuda")
    res = {}
    for gm in ("0", "8"):
        env = {"MOE_GEMM_MAX_BLOCKS": str(blocks), "MOE_GEMM_SPLIT_MIN_STEPS": "0", "MOE_GEMM_GROUP_M": gm}
        os.environ.update(env)
        try:
            _, g = run_train(moe, cfg, inp, dy)
        finally:
            for key in env:
                del os.environ[key]
        res[gm] = {key: g[key].clone() for key in ("dx", "dw_router", "dW1", "dW2")}
    for key in res["0"]:
        assert torch.equal(res["0"][key], res["8"][key]), key


def test_backward_chunked_hot_experts(moe):
    """Skewed routing: the weight-gradient reductions of the two hot experts
    are cut into chunks of K steps whose float32 partial sums a fixup adds in
    chunk order. The gradients match the oracle, repeat bit for bit, and differ
    (in rounding only) from the run that keeps every reduction whole, which
    shows that the chunked path ran."""
    import os
    cfg = scaled_config("skewed", T=2048, d_model=256, E=16, k=4, d_expert=256, suffix="chunk")
    announce("backward chunked hot experts")
    inp = make_inputs(cfg, seed=10, device="cuda")
    dy = make_dense((cfg.T, cfg.d_model), 1.0, seed=10, tag=9, device="cuda")
    runs = {}
    for name, env in (("chunked", {}), ("chunked2", {}), ("whole", {"MOE_BWD_KGROUP_SLOTS": "0"})):
        os.environ.update(env)
        try:
            _, g = run_train(moe, cfg, inp, dy)
        finally:
            for key in env:
                del os.environ[key]
        runs[name] = {key: g[key].clone() for key in ("dx", "dw_router", "dW1", "dW2")}
    for key in runs["chunked"]:
        assert torch.equal(runs["chunked"][key], runs["chunked2"][key]), key
    assert not (torch.equal(runs["chunked"]["dW1"], runs["whole"]["dW1"])
                and torch.equal(runs["chunked"]["dW2"], runs["whole"]["dW2"]))
    h = {kk: host_array(v) for kk, v in inp.items()}
    ref = oracle.backward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype,
                          host_array(dy))
    assert not ref["near_tie"].any()
    for name in ("chunked", "whole"):
        for key in ("dx", "dw_router", "dW1", "dW2"):
            err = rel_err(f64(runs[name][key]), ref[key])
            print(f"{name} {key}: rel err {err:.3e}")
            assert err <= TOL_BF16, (name, key)


def test_backward_repeatable_and_workspace_reuse(moe):
    """Two backward calls on one training workspace give identical results (no
    atomics, fixed summation orders), and a second training step reuses it."""
    cfg = scaled_config("fine_grained", T=200, d_model=256, d_expert=256, suffix="bwd")
    announce("backward repeatable")
    inp = make_inputs(cfg, seed=4, device="cuda")
    dy = make_dense((cfg.T, cfg.d_model), 1.0, seed=4, tag=9, device="cuda")
    _, a = run_train(moe, cfg, inp, dy)
    _, b = run_train(moe, cfg, inp, dy)
    for key in a:
        assert torch.equal(a[key], b[key]), key


FULL = ["mixtral_coarse", "fine_grained", "skewed", "large_sparse"]


def _unsettled_experts(logits32, near_tie, k, margin=1e-6):
    """Experts whose selection a near-tie token could flip: those within `margin`
    of that token's k-th largest float32 logit."""
    out = set()
    for t in np.nonzero(near_tie)[0]:
        row = logits32[t].astype(np.float64)
        lk = np.sort(row)[::-1][k - 1]
        out |= set(np.nonzero(np.abs(row - lk) < margin)[0].tolist())
    return out


def _check_expert_grads(name, got, ref, experts):
    """dW of each listed expert over its whole slice, scaled by that slice's max."""
    for key in ("dW1", "dW2"):
        for e in experts:
            err = rel_err(f64(got[key][e]), ref[key][e] if isinstance(ref[key], np.ndarray) else ref[key](e))
            print(f"{name}: {key}[{e}] rel err {err:.3e}", flush=True)
            assert err <= TOL_BF16, (key, e)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_backward_full_size(moe, name):
    """The workloads at full size, as one training step runs them, against the
    backward oracle: dx of every token outside near-ties, the router weight and
    bias gradients, every expert's dW1 and dW2 (the whole tensors, and whole
    slices of the busiest, a middle and the least used expert with rows, each
    scaled by its own max) and the load statistics. For the large layer (60 GB
    of float64 weight gradients) dx is checked on 1024 tokens (the backward of
    just those tokens: dx is token-local) and dW on the three experts' whole
    slices, each the oracle's per-expert backward over all of its rows."""
    from harness import CONFIGS
    cfg = CONFIGS[name]
    announce(f"backward full {name}")
    inp = make_inputs(cfg, seed=0, device="cuda")
    dy = make_dense((cfg.T, cfg.d_model), 1.0, seed=0, tag=9, device="cuda")
    _, g = run_train(moe, cfg, inp, dy)
    x64 = oracle.decode(host_array(inp["x"]), "bf16")
    wr64 = oracle.decode(host_array(inp["w_router"]), "bf16")
    bias = host_array(inp["router_bias"])
    dy64 = oracle.decode(host_array(dy), "bf16")
    r = oracle.route(x64, wr64, bias, cfg.k)
    counts = np.bincount(r["idx"].reshape(-1), minlength=cfg.E)
    np.testing.assert_allclose(f64(g["load_frac"]), counts / (cfg.T * cfg.k), rtol=1e-6, atol=0)
    np.testing.assert_allclose(f64(g["mean_prob"]), oracle.softmax_probs(r["logits"]).mean(axis=0), rtol=1e-4,
                               atol=1e-7)
    tie = r["near_tie"]
    unsettled = _unsettled_experts(r["logits"], tie, cfg.k)
    used = np.nonzero(counts > 0)[0]
    order = [int(e) for e in used[np.argsort(-counts[used], kind="stable")] if int(e) not in unsettled]
    experts = sorted({order[0], order[len(order) // 2], order[-1]})
    print(f"{name}: near-ties {int(tie.sum())}, experts they could flip {sorted(unsettled)}, "
          f"checked slices {experts} (counts {[int(counts[e]) for e in experts]})", flush=True)
    w1 = lambda e: oracle.decode(host_array(inp["W1"][e]), "bf16")  # noqa: E731
    w2 = lambda e: oracle.decode(host_array(inp["W2"][e]), "bf16")  # noqa: E731

    if name != "large_sparse":
        ref = oracle.backward64(x64, wr64, w1, w2, cfg.k, dy64, r["idx"], r["logits"])
        keep = ~tie
        err = rel_err(f64(g["dx"])[keep], ref["dx"][keep])
        print(f"{name}: dx rel err {err:.3e} over {int(keep.sum())} of {cfg.T} tokens", flush=True)
        assert err <= TOL_BF16
        for key in ("dw_router", "dbias"):
            err = rel_err(f64(g[key]), ref[key])
            print(f"{name}: {key} rel err {err:.3e}", flush=True)
            assert err <= TOL_BF16, key
        settled = np.array([e for e in range(cfg.E) if e not in unsettled])
        for key in ("dW1", "dW2"):
            err = rel_err(f64(g[key][torch.from_numpy(settled).cuda()]), ref[key][settled])
            print(f"{name}: {key} rel err {err:.3e} over {settled.size} experts", flush=True)
            assert err <= TOL_BF16, key
        _check_expert_grads(name, g, ref, experts)
        for e in np.nonzero(counts == 0)[0]:
            assert torch.count_nonzero(g["dW1"][e]) == 0 and torch.count_nonzero(g["dW2"][e]) == 0
        return

    # large layer: dx of 1024 tokens outside near-ties
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(np.nonzero(~tie)[0], 1024, replace=False))
    sub = oracle.backward64(x64[toks], wr64, w1, w2, cfg.k, dy64[toks], r["idx"][toks], r["logits"][toks])
    err = rel_err(f64(g["dx"][torch.from_numpy(toks).cuda()]), sub["dx"])
    print(f"{name}: dx rel err {err:.3e} on {toks.size} tokens", flush=True)
    assert err <= TOL_BF16
    # whole dW slices of three experts: the oracle's per-expert backward over all of their rows
    gate = oracle.softmax_gates(r["logits"], r["idx"])
    ref = {"dW1": {}, "dW2": {}}
    for e in experts:
        sel = np.argwhere(r["idx"] == e)  # (token, slot) in token order
        X = x64[sel[:, 0]]
        dYp = gate[sel[:, 0], sel[:, 1]][:, None] * dy64[sel[:, 0]]
        ge = oracle.expert_backward(X, dYp, w1(e), w2(e))
        ref["dW1"][e], ref["dW2"][e] = ge["dW1"], ge["dW2"]
    _check_expert_grads(name, g, {key: (lambda e, key=key: ref[key][e]) for key in ref}, experts)
