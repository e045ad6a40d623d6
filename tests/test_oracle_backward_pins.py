"""Pins of the backward oracle to facts outside itself (no GPU needed).

The backward oracle writes out the chain rule; these tests check it against
central finite differences of the forward (float64, expert choice held
fixed), against torch's autograd of the same layer written with torch ops,
and against closed forms: GELU_tanh' against its library derivative, softmax
gradients summing to zero per token, the single-expert and identical-expert
cases that reduce to a dense FFN, and the load statistics' sums.
"""

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng


def rand_layer(T, d, E, k, de, seed, bias=True, router_std=0.5):
    g = RNG(seed)
    x = g.standard_normal((T, d))
    wr = g.standard_normal((d, E)) * router_std
    b = g.standard_normal(E) * 0.3 if bias else None
    W1 = g.standard_normal((E, d, de)) * d ** -0.5
    W2 = g.standard_normal((E, de, d)) * de ** -0.5
    dy = g.standard_normal((T, d))
    return x, wr, b, W1, W2, dy


def selection(x, wr, b, k):
    logits = oracle.router_logits(x, wr, b, rounded=False)
    s = -np.sort(-logits, axis=1)
    margin = (s[:, k - 1] - s[:, k]).min() if k < logits.shape[1] else np.inf
    return oracle.topk_select(logits, k), logits, margin


def test_gelu_grad_matches_library_autograd_and_differences():
    u = np.linspace(-9, 9, 3601)
    ut = torch.from_numpy(u).requires_grad_(True)
    torch.nn.functional.gelu(ut, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(u), ut.grad.numpy(), rtol=1e-12, atol=1e-14)
    h = 1e-6
    fd = (oracle.gelu_tanh(u + h) - oracle.gelu_tanh(u - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(u), fd, rtol=1e-6, atol=1e-8)
    assert oracle.gelu_tanh_grad(np.array([0.0]))[0] == 0.5


def test_backward_matches_central_differences():
    """Every parameter and input of a tiny layer: d(sum dy * y)/dtheta by central
    differences of the smooth forward against the backward's gradients."""
    T, d, E, k, de = 5, 6, 4, 2, 7
    x, wr, b, W1, W2, dy = rand_layer(T, d, E, k, de, seed=11)
    idx, logits, margin = selection(x, wr, b, k)
    assert margin > 1e-3  # no selection change under the perturbations below
    g = oracle.backward64(x, wr, W1, W2, k, dy, idx, logits)

    def loss(x_, wr_, b_, W1_, W2_):
        return float(np.sum(dy * oracle.forward64_fixed(x_, wr_, b_, W1_, W2_, idx)))

    h = 1e-6
    params = {"dx": x, "dw_router": wr, "dbias": b, "dW1": W1, "dW2": W2}
    args = [x, wr, b, W1, W2]
    for pos, (name, arr) in enumerate(params.items()):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a_p, a_m = arr.copy(), arr.copy()
            a_p[i] += h
            a_m[i] -= h
            ap, am = list(args), list(args)
            ap[pos], am[pos] = a_p, a_m
            fd[i] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def torch_layer_grads(x, wr, b, W1, W2, dy, idx):
    """The same layer with torch ops and autograd (float64), expert choice fixed."""
    tx, twr, tb, tW1, tW2 = (torch.tensor(a, requires_grad=True) for a in (x, wr, b, W1, W2))
    p = torch.softmax(tx @ twr + tb, dim=1)
    T, k = idx.shape
    y = torch.zeros_like(tx)
    for j in range(k):
        e = torch.from_numpy(idx[:, j].astype(np.int64))
        h = torch.nn.functional.gelu(torch.bmm(tx[:, None, :], tW1[e]), approximate="tanh")
        yj = torch.bmm(h, tW2[e])[:, 0, :]
        y = y + p[torch.arange(T), e][:, None] * yj
    (y * torch.from_numpy(dy)).sum().backward()
    return {"dx": tx.grad.numpy(), "dw_router": twr.grad.numpy(), "dbias": tb.grad.numpy(),
            "dW1": tW1.grad.numpy(), "dW2": tW2.grad.numpy()}


@pytest.mark.parametrize("T,d,E,k,de,seed", [(40, 16, 6, 2, 24, 1), (33, 8, 8, 8, 12, 2), (50, 12, 5, 1, 16, 3)])
def test_backward_matches_torch_autograd(T, d, E, k, de, seed):
    x, wr, b, W1, W2, dy = rand_layer(T, d, E, k, de, seed)
    idx, logits, _ = selection(x, wr, b, k)
    g = oracle.backward64(x, wr, W1, W2, k, dy, idx, logits)
    ref = torch_layer_grads(x, wr, b, W1, W2, dy, idx)
    for name, v in ref.items():
        np.testing.assert_allclose(g[name], v, rtol=1e-10, atol=1e-12, err_msg=name)


def test_softmax_gradient_sums_to_zero_and_statistics_sum_to_one():
    T, d, E, k, de = 64, 16, 8, 3, 20
    x, wr, b, W1, W2, dy = rand_layer(T, d, E, k, de, seed=4)
    idx, logits, _ = selection(x, wr, b, k)
    g = oracle.backward64(x, wr, W1, W2, k, dy, idx, logits)
    np.testing.assert_allclose(g["dlogit"].sum(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dbias"].sum(), 0.0, atol=1e-12)
    assert abs(g["load_frac"].sum() - 1.0) < 1e-15 and abs(g["mean_prob"].sum() - 1.0) < 1e-14
    assert np.all(g["load_frac"] * T * k == np.bincount(idx.reshape(-1), minlength=E))


def dense_ffn_grads(x, w1, w2, dy):
    tx, t1, t2 = (torch.tensor(a, requires_grad=True) for a in (x, w1, w2))
    y = torch.nn.functional.gelu(tx @ t1, approximate="tanh") @ t2
    (y * torch.from_numpy(dy)).sum().backward()
    return tx.grad.numpy(), t1.grad.numpy(), t2.grad.numpy()


def test_single_expert_is_dense_ffn_backward():
    """E = k = 1: the gate is 1, no router gradient, and the rest is the dense FFN's backward."""
    x, wr, b, W1, W2, dy = rand_layer(20, 8, 1, 1, 12, seed=5)
    idx, logits, _ = selection(x, wr, b, 1)
    g = oracle.backward64(x, wr, W1, W2, 1, dy, idx, logits)
    assert np.all(g["dlogit"] == 0) and np.all(g["dw_router"] == 0)
    dx, d1, d2 = dense_ffn_grads(x, W1[0], W2[0], dy)
    np.testing.assert_allclose(g["dx"], dx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dW1"][0], d1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dW2"][0], d2, rtol=1e-12, atol=1e-13)


def test_identical_experts_with_k_equal_E_is_dense_ffn_backward():
    """All E experts identical and all selected: y = FFN(x) whatever the router,
    so the router gets no gradient and each expert gets its gate's share."""
    T, d, E, de = 16, 8, 4, 10
    x, wr, b, W1, W2, dy = rand_layer(T, d, E, E, de, seed=6)
    W1[:] = W1[0]
    W2[:] = W2[0]
    idx, logits, _ = selection(x, wr, b, E)
    g = oracle.backward64(x, wr, W1, W2, E, dy, idx, logits)
    dx, d1, d2 = dense_ffn_grads(x, W1[0], W2[0], dy)
    np.testing.assert_allclose(g["dlogit"], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dx"], dx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dW1"].sum(axis=0), d1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dW2"].sum(axis=0), d2, rtol=1e-11, atol=1e-12)


def test_unused_expert_gets_zero_weight_gradient_and_zero_dy_gives_zero():
    T, d, E, k, de = 12, 8, 6, 1, 10
    x, wr, b, W1, W2, dy = rand_layer(T, d, E, k, de, seed=7)
    b[5] = -1e3  # expert 5 is never selected
    idx, logits, _ = selection(x, wr, b, k)
    assert not np.any(idx == 5)
    g = oracle.backward64(x, wr, W1, W2, k, dy, idx, logits)
    assert np.all(g["dW1"][5] == 0) and np.all(g["dW2"][5] == 0)
    z = oracle.backward64(x, wr, W1, W2, k, np.zeros_like(dy), idx, logits)
    for name in ("dx", "dw_router", "dbias", "dW1", "dW2"):
        assert np.all(z[name] == 0), name


def test_backward_on_workload_arrays_routes_like_the_forward():
    """The raw-array entry point (bf16 bit patterns) selects exactly the experts
    of the forward oracle and differentiates at its float32 logits."""
    from harness import make_inputs, scaled_config, to_host_arrays
    cfg = scaled_config("fine_grained", T=48, d_model=64, E=16, k=4, d_expert=32)
    h = to_host_arrays(make_inputs(cfg, seed=3, device="cpu"))
    dy = h["x"][::-1].copy()
    f = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    g = oracle.backward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype, dy)
    assert np.array_equal(g["idx"], f["idx"])
    np.testing.assert_allclose(g["gate"], f["gate"], rtol=1e-15)
    np.testing.assert_allclose(g["Y"], f["Y_perm"], rtol=1e-12, atol=1e-14)
