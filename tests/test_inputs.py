"""The seeded input generator: reproducible, right shapes, dtypes and spreads."""

import numpy as np
import torch

from harness import CONFIGS, make_inputs, scaled_config, to_host_arrays
from harness.configs import CONFIG_ORDER


def test_same_seed_same_bytes_and_seed_changes_values():
    cfg = scaled_config("fine_grained", T=64, d_model=64, E=8, k=2, d_expert=64)
    a = to_host_arrays(make_inputs(cfg, seed=0))
    b = to_host_arrays(make_inputs(cfg, seed=0))
    c = to_host_arrays(make_inputs(cfg, seed=1))
    for key in ("x", "w_router", "W1", "W2"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


def test_shapes_dtypes_and_bias_of_every_workload():
    for name in CONFIG_ORDER:
        cfg = CONFIGS[name]
        small = scaled_config(name, T=32, d_model=64, d_expert=64)
        inp = make_inputs(small, seed=0)
        dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        assert inp["x"].shape == (32, 64) and inp["x"].dtype == dt
        assert inp["w_router"].shape == (64, cfg.E) and inp["w_router"].dtype == dt
        assert inp["W1"].shape == (cfg.E, 64, 64) and inp["W2"].shape == (cfg.E, 64, 64)
        assert (inp["router_bias"] is not None) == (name == "skewed")
    b = make_inputs(scaled_config("skewed", T=8, d_model=64, d_expert=64), seed=0)["router_bias"]
    want = np.zeros(64, dtype=np.float32)
    want[[0, 1]] = 3.0
    want[60:64] = -6.0
    assert np.array_equal(b.numpy(), want)


def test_standard_deviations_follow_the_fan_in_reading():
    cfg = scaled_config("mixtral_coarse", T=256, d_model=512, E=2, k=1, d_expert=1024)
    inp = make_inputs(cfg, seed=0)
    def std(t):
        return float(t.float().std())
    assert abs(std(inp["x"]) - 1.0) < 0.02
    assert abs(std(inp["w_router"]) - 0.02) < 0.002
    assert abs(std(inp["W1"]) * 512 ** 0.5 - 1.0) < 0.02
    assert abs(std(inp["W2"]) * 1024 ** 0.5 - 1.0) < 0.02


def test_bf16_rounding_is_nearest_even():
    # the generator rounds float32 to bf16 through torch's conversion; pin its rounding
    vals = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -(1.0 + 2 ** -8)],
                        dtype=torch.float32)
    got = vals.to(torch.bfloat16).float().tolist()
    assert got == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0]


def test_router_zero_inputs():
    cfg = scaled_config("skewed", T=8, d_model=64, d_expert=64)
    inp = make_inputs(cfg, router_zero=True)
    assert torch.count_nonzero(inp["w_router"]) == 0
    assert torch.count_nonzero(inp["router_bias"]) == 0
