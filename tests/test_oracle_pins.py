"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something it does not compute itself:
brute-force enumeration, exact special cases, reductions to library routines
(torch's GELU, softmax and matmul in float64), invariants that any correct
implementation satisfies, and the worked number printed on the source page.
"""

import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from harness import make_inputs, scaled_config, to_host_arrays
from harness.configs import MoEConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(T=24, d=32, E=6, k=2, de=48, dtype="f32", bias=None):
    return MoEConfig("t", T=T, d_model=d, E=E, k=k, d_expert=de, dtype=dtype,
                     x_std=1.0, router_std=0.5, w1_std=d ** -0.5, w2_std=de ** -0.5,
                     router_bias=bias)


def host_inputs(cfg, seed=0, router_zero=False):
    return to_host_arrays(make_inputs(cfg, seed=seed, device="cpu", router_zero=router_zero))


def dense_ffn_torch(x64, w1, w2):
    """Dense FFN with library routines only: torch matmul and torch's tanh GELU (float64)."""
    h = torch.nn.functional.gelu(torch.from_numpy(x64) @ torch.from_numpy(w1), approximate="tanh")
    return (h @ torch.from_numpy(w2)).numpy()


# --------------------------------------------------------------------------- decoding

def test_decode_bf16_golden_bits():
    cases = json.load(open(os.path.join(GOLDEN, "bf16_bits.json")))["cases"]
    bits = np.array([int(h, 16) for h, _ in cases], dtype=np.uint16)
    vals = oracle.decode(bits, "bf16")
    for (h, v), got in zip(cases, vals):
        assert got == v and np.signbit(got) == np.signbit(v), h


def test_decode_f32_is_exact():
    a = np.array([1.5, -3.25e-20, 7e30], dtype=np.float32)
    assert np.array_equal(oracle.decode(a, "f32"), a.astype(np.float64))


# --------------------------------------------------------------------------- router

def test_router_logits_exact_integer_case():
    # x = ones, Wr[c, e] = c + e  ->  logit[e] = sum_c (c + e) = d(d-1)/2 + d*e, exact in float32
    d, E = 16, 5
    x = np.ones((3, d))
    wr = np.add.outer(np.arange(d), np.arange(E)).astype(np.float64)
    b = np.array([0.5, 0, 0, -1, 0], dtype=np.float32)
    got = oracle.router_logits(x, wr, b)
    want = np.array([d * (d - 1) / 2 + d * e for e in range(E)]) + b
    assert got.dtype == np.float32
    assert np.array_equal(got, np.tile(want.astype(np.float32), (3, 1)))


def test_router_logits_round_once_to_float32():
    # 1 + 2^-30 is not a float32; the float64 sum rounds once to 1.0
    x = np.array([[1.0, 2.0 ** -30]])
    wr = np.array([[1.0], [1.0]])
    assert oracle.router_logits(x, wr, None)[0, 0] == np.float32(1.0)


def _brute_topk_set(l, k):
    """The unique k-subset S with: for i in S, j not in S, l_i > l_j or (l_i == l_j and i < j)."""
    E = len(l)
    found = []
    for S in itertools.combinations(range(E), k):
        ok = all((l[i] > l[j]) or (l[i] == l[j] and i < j)
                 for i in S for j in range(E) if j not in S)
        if ok:
            found.append(set(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("E,k", [(2, 1), (3, 2), (5, 1), (6, 3), (8, 2), (8, 4), (12, 4), (7, 7)])
def test_topk_matches_brute_force_enumeration(E, k):
    rng = np.random.default_rng(E * 31 + k)
    # quantised logits so that exact ties are frequent
    logits = (rng.integers(-3, 4, size=(200, E)) * 0.25).astype(np.float32)
    logits[0] = 0.0
    logits[1, :] = -0.0
    logits[1, ::2] = 0.0
    idx = oracle.topk_select(logits, k)
    for t in range(logits.shape[0]):
        l = logits[t].astype(np.float64)
        assert set(idx[t].tolist()) == _brute_topk_set(l, k)
        for j in range(k - 1):  # order: descending logit, ties to the lower index
            a, b = idx[t, j], idx[t, j + 1]
            assert l[a] > l[b] or (l[a] == l[b] and a < b)


def test_softmax_gates_match_library_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 9)).astype(np.float32) * 4
    idx = oracle.topk_select(logits, 3)
    gate = oracle.softmax_gates(logits, idx)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(gate, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=1e-14)


def test_near_ties_margin():
    logits = np.array([[1.0, 0.5, 0.5 - 5e-7, 0.0],
                       [1.0, 0.5, 0.5 - 2e-6, 0.0],
                       [1.0, 0.5, 0.5, 0.0]], dtype=np.float32)
    assert oracle.near_ties(logits, 2).tolist() == [True, False, True]
    assert not oracle.near_ties(logits, 4).any()


# --------------------------------------------------------------------------- special cases

def test_zero_router_tie_break_and_uniform_gates():
    cfg = tiny_cfg(E=8, k=3)
    h = host_inputs(cfg, router_zero=True)
    out = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    assert np.all(out["logits"] == 0)
    assert np.array_equal(out["idx"], np.tile(np.arange(3, dtype=np.int32), (cfg.T, 1)))
    assert np.all(out["gate"] == 1.0 / 8)
    x64 = h["x"].astype(np.float64)
    want = sum(dense_ffn_torch(x64, h["W1"][e].astype(np.float64), h["W2"][e].astype(np.float64))
               for e in range(3)) / 8
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-14)


def test_k_equals_E_identical_experts_is_dense_ffn():
    cfg = tiny_cfg(E=5, k=5)
    h = host_inputs(cfg)
    W1 = np.repeat(h["W1"][:1], cfg.E, axis=0)
    W2 = np.repeat(h["W2"][:1], cfg.E, axis=0)
    out = oracle.forward(h["x"], h["w_router"], None, W1, W2, cfg.k, cfg.dtype)
    np.testing.assert_allclose(out["gate"].sum(axis=1), 1.0, rtol=1e-14)
    want = dense_ffn_torch(h["x"].astype(np.float64), W1[0].astype(np.float64), W2[0].astype(np.float64))
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-13)


def test_single_expert_top1_is_dense_ffn_bf16():
    cfg = tiny_cfg(E=1, k=1, dtype="bf16")
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], None, h["W1"], h["W2"], 1, "bf16")
    assert np.all(out["gate"] == 1.0)
    x64 = oracle.decode(h["x"], "bf16")
    want = dense_ffn_torch(x64, oracle.decode(h["W1"], "bf16")[0], oracle.decode(h["W2"], "bf16")[0])
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- GELU

def test_gelu_matches_library_and_closed_forms():
    u = np.linspace(-8, 8, 2001)
    g = oracle.gelu_tanh(u)
    lib = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(g, lib, rtol=1e-14, atol=1e-15)
    # odd part of x*Phi-like forms: GELU(u) - GELU(-u) = u
    np.testing.assert_allclose(g - oracle.gelu_tanh(-u), u, rtol=1e-13, atol=1e-14)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert oracle.gelu_tanh(np.array([10.0]))[0] == 10.0
    assert oracle.gelu_tanh(np.array([-10.0]))[0] == 0.0
    # small-u slope 1/2: GELU(u) = u/2 + sqrt(2/pi) u^2 / 2 + O(u^4)
    s = 1e-4
    np.testing.assert_allclose(oracle.gelu_tanh(np.array([s]))[0],
                               s / 2 + np.sqrt(2 / np.pi) * s * s / 2, rtol=1e-7)


# --------------------------------------------------------------------------- dispatch invariants

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 4, 2), (100, 16, 4), (33, 8, 8)])
def test_permutation_invariants(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    p = oracle.permute(idx, E)
    counts, offsets, perm, inv = p["counts"], p["offsets"], p["perm"], p["inv"]
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[E] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    flat = idx.reshape(-1)
    for i in range(T * k):
        r = inv[i]
        assert perm[r] == i // k  # row r holds token t of selection (t, j)
        assert offsets[flat[i]] <= r < offsets[flat[i] + 1]  # inside its expert's group
    assert sorted(inv.tolist()) == list(range(T * k))
    for e in range(E):
        toks = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(toks) > 0)  # token order, each token at most once per expert
    assert np.array_equal(np.bincount(perm, minlength=T), np.full(T, k))


def test_permute_empty_groups():
    idx = np.array([[3, 0], [0, 3], [3, 0]], dtype=np.int32)
    p = oracle.permute(idx, 6)
    assert p["counts"].tolist() == [3, 0, 0, 3, 0, 0]
    assert p["offsets"].tolist() == [0, 3, 3, 3, 6, 6, 6]
    assert p["perm"].tolist() == [0, 1, 2, 0, 1, 2]
    assert p["inv"].tolist() == [3, 0, 1, 4, 5, 2]


def test_active_fraction_page_value():
    g = json.load(open(os.path.join(GOLDEN, "active_fraction.json")))
    cfg = tiny_cfg(T=40, E=g["E"], k=g["k"])
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], None, h["W1"], h["W2"], cfg.k, cfg.dtype)
    # each token's row is multiplied by the weights of k of the E experts
    used = out["counts"].sum() / (cfg.T * cfg.E)
    assert used == g["active_fraction"]
    assert cfg.ffn_flops() == g["active_fraction"] * 4 * cfg.T * cfg.E * cfg.d_model * cfg.d_expert


# --------------------------------------------------------------------------- whole-layer pins

def test_dense_masked_formulation_agrees():
    """Independent formulation: every expert on every token (torch), masked by the brute-force top-k set."""
    cfg = tiny_cfg(T=20, d=24, E=6, k=3, de=40, bias=((1, 0.7), (4, -0.3)))
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    x = torch.from_numpy(h["x"].astype(np.float64))
    logits = (x @ torch.from_numpy(h["w_router"].astype(np.float64))
              + torch.from_numpy(h["router_bias"].astype(np.float64))).float()
    assert np.array_equal(logits.numpy(), out["logits"])
    p = torch.softmax(logits.double(), dim=1).numpy()
    y = np.zeros((cfg.T, cfg.d_model))
    for t in range(cfg.T):
        S = _brute_topk_set(logits[t].double().numpy(), cfg.k)
        for e in S:
            y[t] += p[t, e] * dense_ffn_torch(h["x"][t:t + 1].astype(np.float64),
                                              h["W1"][e].astype(np.float64), h["W2"][e].astype(np.float64))[0]
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-13)


def test_literal_form_equals_batched_form():
    cfg = scaled_config("tiny_fp32", T=32)
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], None, h["W1"], h["W2"], cfg.k, cfg.dtype)
    lit = oracle.forward_literal(h["x"], h["w_router"], None, h["W1"], h["W2"], cfg.k, cfg.dtype)
    np.testing.assert_allclose(out["y"], lit, rtol=1e-12, atol=1e-13)


def test_forward_tokens_equals_full_forward_rows():
    cfg = tiny_cfg(T=30, E=8, k=2, dtype="bf16", bias=((0, 1.0),))
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, "bf16")
    rows = np.array([0, 7, 29])
    sub = oracle.forward_tokens(h["x"][rows], h["w_router"], h["router_bias"],
                                lambda e: h["W1"][e], lambda e: h["W2"][e], cfg.k, "bf16")
    np.testing.assert_allclose(sub["y"], out["y"][rows], rtol=1e-12, atol=1e-13)
    assert np.array_equal(sub["idx"], out["idx"][rows])


def test_token_permutation_equivariance():
    cfg = tiny_cfg(T=25, E=7, k=2)
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], None, h["W1"], h["W2"], cfg.k, cfg.dtype)
    sig = np.random.default_rng(1).permutation(cfg.T)
    out2 = oracle.forward(h["x"][sig], h["w_router"], None, h["W1"], h["W2"], cfg.k, cfg.dtype)
    assert np.array_equal(out2["idx"], out["idx"][sig])
    np.testing.assert_allclose(out2["y"], out["y"][sig], rtol=1e-13, atol=1e-14)


def test_expert_relabeling_invariance():
    cfg = tiny_cfg(T=25, E=7, k=3, bias=((2, 0.4),))
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], h["router_bias"], h["W1"], h["W2"], cfg.k, cfg.dtype)
    assert not out["near_tie"].any()
    pi = np.random.default_rng(5).permutation(cfg.E)  # new expert e' = position of old expert
    wr2 = h["w_router"][:, pi]
    b2 = h["router_bias"][pi]
    out2 = oracle.forward(h["x"], wr2, b2, h["W1"][pi], h["W2"][pi], cfg.k, cfg.dtype)
    np.testing.assert_allclose(out2["y"], out["y"], rtol=1e-13, atol=1e-14)
    assert np.array_equal(pi[out2["idx"]], out["idx"])


def test_linearity_in_W2():
    cfg = tiny_cfg(T=16, E=4, k=2, dtype="bf16")
    h = host_inputs(cfg)
    out = oracle.forward(h["x"], h["w_router"], None, h["W1"], h["W2"], cfg.k, "bf16")
    assert np.all((h["W2"] & 0x7F80) != 0)  # all normal numbers: +1 in the exponent field doubles
    W2x2 = (h["W2"].astype(np.uint32) + (1 << 7)).astype(np.uint16)
    out2 = oracle.forward(h["x"], h["w_router"], None, h["W1"], W2x2, cfg.k, "bf16")
    assert np.array_equal(out2["y"], 2 * out["y"])
