"""The whole layer on the GPU against the oracle, element by element.

Every workload runs twice: at an oracle-sized scale (intermediates included)
and at its full size in the launch configuration the benchmark times
(moe_forward on one stream). Both are compared over every token:

  * R-exact: the oracle's selection and dispatch (top-k by (-logit, index),
    stable grouping by expert) applied to the GPU's own float32 logits must
    give the GPU's idx, counts, offsets, perm and inv bit for bit. With
    identical logits the total order leaves exactly one correct result, so
    nothing is excluded here;
  * R-logits: the GPU's logits lie within the float32 dot-product rounding
    bound of the exact ones;
  * R-e2e: the GPU selects the oracle's expert set for every token outside the
    oracle's near-ties (k-th minus (k+1)-th float32 logit below 1e-6); near-tie
    tokens are reported and left out of the output comparison;
  * Y: max|y_gpu - y_ref| / max|y_ref| over every remaining element, within
    1e-2 for bf16 and 1e-5 for float32.

The oracle is token-local, so the full-size reference is computed over token
chunks (the routing, dispatch, experts and combine of the chunk's tokens),
with the expert weights streamed one expert at a time.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL_BF16, TOL_F32, announce, check_routing_e2e, check_routing_exact, f64, needs_gpu,
                         rel_err)
from harness import CONFIGS, host_array, make_inputs, scaled_config
from harness.configs import CONFIG_ORDER

pytestmark = [pytest.mark.gpu, needs_gpu]

SMALL = {
    "tiny_fp32": dict(),
    "mixtral_coarse": dict(T=512, d_model=512, d_expert=1024),
    "fine_grained": dict(T=640, d_model=256, d_expert=256),
    "skewed": dict(T=1000, d_model=256, d_expert=256),
    "large_sparse": dict(T=300, d_model=512, d_expert=256),
}


def tol(cfg):
    return TOL_F32 if cfg.dtype == "f32" else TOL_BF16


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_forward_small_all_stages(moe, name):
    cfg = scaled_config(name, **SMALL[name]) if SMALL[name] else CONFIGS[name]
    announce(f"forward small {cfg.name} T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k} de={cfg.d_expert}")
    inp = make_inputs(cfg, seed=0, device="cuda")
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    st = layer.stages(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    y_fwd = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(y_fwd, st["y"]), "moe_forward and the four stage calls must agree bitwise"

    h = {k: host_array(v) for k, v in inp.items()}
    ref = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    logits, idx, pm = check_routing_exact(cfg, st)
    x64, wr64 = oracle.decode(h["x"], cfg.dtype), oracle.decode(h["w_router"], cfg.dtype)
    keep = check_routing_e2e(cfg, logits, idx, f64(st["gate"]), x64, wr64, h["router_bias"], ref)
    # the permuted copy is the oracle's gather of the GPU's own dispatch
    assert np.array_equal(f64(st["x_perm"]), oracle.gather_rows(x64, pm["perm"]))
    err = rel_err(f64(st["y"])[keep], ref["y"][keep])
    print(f"{cfg.name}: y rel err {err:.3e} over {int(keep.sum())} of {cfg.T} tokens, "
          f"counts min/max {ref['counts'].min()}/{ref['counts'].max()}")
    assert err <= tol(cfg)


CHUNK = 8192  # tokens per oracle call at full size


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_forward_full_size_every_token(moe, name):
    cfg = CONFIGS[name]
    announce(f"forward full {name} T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k} de={cfg.d_expert}")
    inp = make_inputs(cfg, seed=0, device="cuda")
    layer = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, inp["x"].dtype)
    y = layer(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"]).clone()
    st = layer.stages(inp["x"], inp["w_router"], inp["W1"], inp["W2"], inp["router_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y, st["y"]), "moe_forward and the four stage calls must agree bitwise"
    got = f64(y)
    gate = f64(st["gate"])
    logits, idx, _ = check_routing_exact(cfg, st)
    for key in ("x_perm", "y_perm", "y"):
        st[key] = None
    del y
    torch.cuda.empty_cache()

    xh, wrh, bh = host_array(inp["x"]), host_array(inp["w_router"]), host_array(inp["router_bias"])
    W1, W2 = inp["W1"], inp["W2"]
    w1h = [host_array(W1[e]) for e in range(cfg.E)]
    w2h = [host_array(W2[e]) for e in range(cfg.E)]
    x64, wr64 = oracle.decode(xh, cfg.dtype), oracle.decode(wrh, cfg.dtype)
    ref_route = oracle.route(x64, wr64, bh, cfg.k)
    keep = check_routing_e2e(cfg, logits, idx, gate, x64, wr64, bh, ref_route)
    del x64

    y_ref = np.empty((cfg.T, cfg.d_model), dtype=np.float64)
    for t0 in range(0, cfg.T, CHUNK):
        t1 = min(cfg.T, t0 + CHUNK)
        out = oracle.forward(xh[t0:t1], wrh, bh, lambda e: w1h[e], lambda e: w2h[e], cfg.k, cfg.dtype)
        y_ref[t0:t1] = out["y"]
        del out
        print(f"{name}: oracle tokens {t0}..{t1} done", flush=True)
    err = rel_err(got[keep], y_ref[keep])
    print(f"{name} full size: y rel err {err:.3e} over {int(keep.sum())} of {cfg.T} tokens "
          f"(near-ties excluded {int((~keep).sum())})", flush=True)
    assert err <= tol(cfg)
