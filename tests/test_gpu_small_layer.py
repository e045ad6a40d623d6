"""moe_forward on small float32 problems runs the whole layer as one launch
(one workgroup per token). Its y must be the same bits as the multi-launch
path (route -> permute -> grouped FFN -> combine, forced with
MOE_SMALL_LAYER=0) and match the oracle over every token, for the tiny
workload and for ragged shapes: E not a multiple of 8, k = E, 256 experts,
a single token, wide rows.
"""

import os

import pytest
import torch

import oracle
from gpu_helpers import TOL_F32, announce, check_routing_e2e, check_routing_exact, f64, needs_gpu, rel_err
from harness import host_array, make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [
    # T, d_model, E, k, d_expert
    (64, 128, 8, 2, 256),      # the tiny workload's shape
    (1, 64, 1, 1, 64),
    (37, 192, 13, 5, 320),
    (60, 256, 64, 8, 128),
    (8, 1024, 4, 2, 128),
    (2, 64, 32, 32, 64),       # k = E
    (3, 64, 256, 16, 64),
]


@pytest.mark.parametrize("T,d,E,k,de", CASES, ids=lambda v: str(v))
def test_one_launch_layer_matches_the_staged_path_and_the_oracle(moe, T, d, E, k, de):
    announce(f"small layer T={T} d={d} E={E} k={k} de={de}")
    cfg = scaled_config("tiny_fp32", T=T, d_model=d, E=E, k=k, d_expert=de, suffix="small_layer")
    inp = make_inputs(cfg, seed=31, device="cuda")
    x, wr, b, W1, W2 = inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"]
    p = moe.make_problem(T, d, E, k, de, x.dtype)
    assert moe.moe_plan(p)["forward_one_launch"] == 1
    layer = moe.MoEForward(T, d, E, k, de, x.dtype)
    y1 = layer(x, wr, W1, W2, b).clone()
    y1b = layer(x, wr, W1, W2, b).clone()
    os.environ["MOE_SMALL_LAYER"] = "0"
    try:
        assert moe.moe_plan(p)["forward_one_launch"] == 0
        y8 = layer(x, wr, W1, W2, b).clone()
        st = layer.stages(x, wr, W1, W2, b)
    finally:
        del os.environ["MOE_SMALL_LAYER"]
    torch.cuda.synchronize()
    assert torch.equal(y1, y1b)
    assert torch.equal(y1, y8), "one launch and the staged launches must agree bit for bit"
    assert torch.equal(y1, st["y"])

    ref = oracle.forward_tokens(host_array(x), host_array(wr), host_array(b), lambda e: host_array(W1[e]),
                                lambda e: host_array(W2[e]), k, "f32")
    logits, idx, _ = check_routing_exact(cfg, st)
    keep = check_routing_e2e(cfg, logits, idx, f64(st["gate"]), f64(x), f64(wr), host_array(b), ref)
    err = rel_err(f64(y1)[keep], ref["y"][keep])
    print(f"small layer T={T} d={d} E={E} k={k} de={de}: rel err {err:.3e}, near-ties excluded {int((~keep).sum())}")
    assert err <= TOL_F32


def test_larger_float32_layers_keep_the_staged_launches(moe):
    """Past the size bounds (multiply-adds, or load rounds per thread) the
    one-launch form is not used."""
    assert moe.moe_plan(moe.make_problem(4096, 1024, 8, 2, 1024, "f32"))["forward_one_launch"] == 0
    assert moe.moe_plan(moe.make_problem(4, 1024, 8, 2, 1024, "f32"))["forward_one_launch"] == 0
    assert moe.moe_plan(moe.make_problem(64, 128, 8, 2, 256, "bf16"))["forward_one_launch"] == 0
