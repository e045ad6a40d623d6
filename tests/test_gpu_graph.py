"""moe_forward captured in a HIP graph (through torch.cuda.graph) and
replayed: every launch of the layer goes on the capturing stream, and nothing
is recorded that replays differently from an eager call (the split-tile
counters are cleared by a kernel, not a memset). Each case replays the graph
several times with new inputs copied in and eager work between the replays,
and compares every replay bit for bit with an eager call on the same inputs.
"""

import pytest
import torch

from gpu_helpers import announce, needs_gpu
from harness import make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = [
    # workload, T, d_model, E, k, d_expert (None: the workload's)
    ("mixtral_coarse", 8, None, None, None, None),     # decode: split router fused into the permute, 32-row tile
    ("mixtral_coarse", 32, None, None, None, None),    # decode with the router's finalize launch
    ("skewed", 600, 512, 16, 4, 320),                  # multi-block permute, 256 x 256 tiles
    ("tiny_fp32", None, None, None, None, None),       # float32 one-launch layer
]


@pytest.mark.parametrize("name,T,d,E,k,de", CASES, ids=lambda v: str(v))
def test_forward_replays_in_a_graph(moe, name, T, d, E, k, de):
    cfg = scaled_config(name, T=T, d_model=d, E=E, k=k, d_expert=de, suffix="graph")
    announce(f"graph replay {cfg.name} T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k} de={cfg.d_expert}")
    inputs = [make_inputs(cfg, seed=40 + i, device="cuda") for i in range(3)]
    base = inputs[0]
    x = base["x"].clone()
    wr, b, W1, W2 = base["w_router"], base["router_bias"], base["W1"], base["W2"]
    captured = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, x.dtype)
    eager = moe.MoEForward(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_expert, x.dtype)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            captured(x, wr, W1, W2, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_graph = captured(x, wr, W1, W2, b)
    torch.cuda.synchronize()

    for i in [1, 2, 0, 1]:
        x.copy_(inputs[i]["x"])          # new tokens into the captured input buffer
        junk = torch.randn(4096, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        y_eager = eager(inputs[i]["x"], wr, W1, W2, b)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), f"replay with inputs {i}"
        assert torch.isfinite(junk)
