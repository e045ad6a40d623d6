"""Plain, slow CPU oracle of the sparse MoE layer backward (NumPy, float64).

TEST INFRASTRUCTURE ONLY, like the forward oracle: imported by tests, never
by the product path.

The layer is the forward of moe_oracle: y[t] = sum over j < k of
g[t, j] E_{e(t, j)}(x[t]), with g the softmax probability over all E router
logits of the selected expert ("Distributed training part 4", jesamkim's AI
tech blog, section 3, structure) and E_e(x) = GELU_tanh(x W1_e) W2_e. Given
dy = dL/dy this module writes out the chain rule for every input, step by
step, in the forward's order reversed:

  combine     dYp[r] = g[t, j] dy[t] for the row r of selection (t, j);
              dG[t, j] = dy[t] . Y[r] (Y = the expert output before gating)
  experts     per expert e over its rows: U = X W1_e, H = GELU_tanh(U),
              dH = dYp W2_e^T, dU = dH * GELU_tanh'(U), dX = dU W1_e^T,
              dW2_e = H^T dYp, dW1_e = X^T dU (zero for an expert with no rows)
  dispatch    dx[t] += sum over j of dX[row of (t, j)]
  router      p = softmax of the logits; dp[t, e] = sum of dG[t, j] over the
              j that selected e; dlogit = p * (dp - sum_e p dp) (softmax
              Jacobian); dx += dlogit W_r^T, dW_r = x^T dlogit,
              dbias = sum over tokens of dlogit

The top-k selection is piecewise constant in the logits: no gradient flows
through the choice of experts, only through the gate values.

Router load statistics, the ingredients of a load-balancing loss (the blog's
section on expert collapse motivates one; the pages give no formula, so only
the ingredients are computed): load_frac[e] = counts[e] / (T k), the share of
the T k selections that went to e, and mean_prob[e] = mean over tokens of
p[t, e].
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from .moe_oracle import (WeightSource, _slice, decode, gather_rows, gelu_tanh, permute, route, router_logits,
                         softmax_probs)

_C = math.sqrt(2.0 / math.pi)
_A = 0.044715


def gelu_tanh_grad(u: np.ndarray) -> np.ndarray:
    """d/du of u/2 (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3):
    (1 + tanh z)/2 + u/2 (1 - tanh^2 z) sqrt(2/pi) (1 + 3 * 0.044715 u^2)."""
    u = np.asarray(u, dtype=np.float64)
    th = np.tanh(_C * (u + _A * u * u * u))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * _C * (1.0 + 3.0 * _A * u * u)


def expert_backward(X: np.ndarray, dYp: np.ndarray, w1e: np.ndarray, w2e: np.ndarray) -> Dict[str, np.ndarray]:
    """One expert's forward (recomputed) and backward over its rows, float64.

    X [rows, d] are the expert's input rows, dYp [rows, d] the gradients of its
    gated outputs (g dy of each row's token): U = X W1_e, H = GELU_tanh(U),
    Y = H W2_e, dH = dYp W2_e^T, dU = dH * GELU_tanh'(U), dX = dU W1_e^T,
    dW2_e = H^T dYp (a sum over the rows), dW1_e = X^T dU."""
    U = X @ w1e
    H = gelu_tanh(U)
    dH = dYp @ w2e.T
    dU = dH * gelu_tanh_grad(U)
    return {"U": U, "H": H, "Y": H @ w2e, "dU": dU, "dX": dU @ w1e.T, "dW1": X.T @ dU, "dW2": H.T @ dYp}


def backward64(x64: np.ndarray, wr64: np.ndarray, W1: WeightSource, W2: WeightSource, k: int,
               dy64: np.ndarray, idx: np.ndarray, logits: np.ndarray) -> Dict[str, np.ndarray]:
    """The backward on float64 arrays, for a given selection `idx` [T, k] and the
    logits [T, E] (bias included) the gates come from: float32-rounded for the
    layer as run, float64 for the smooth function. W1/W2: float64 [E, ...] or
    callables e -> slice."""
    T, d = x64.shape
    E = wr64.shape[1]
    R = T * k
    p = softmax_probs(logits)
    gate = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    pm = permute(idx, E)
    inv = pm["inv"].reshape(T, k).astype(np.int64)
    offsets = pm["offsets"]
    xp = gather_rows(x64, pm["perm"])

    # experts forward (recomputed) and backward, one expert at a time
    dYp = np.zeros((R, d), dtype=np.float64)
    for j in range(k):
        dYp[inv[:, j]] = gate[:, j:j + 1] * dy64
    Y = None
    dXp = np.zeros((R, d), dtype=np.float64)
    dW1: Dict[int, np.ndarray] = {}
    dW2: Dict[int, np.ndarray] = {}
    U_all = H_all = dU_all = None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        w1e, w2e = _slice(W1, e), _slice(W2, e)
        de = w1e.shape[1]
        if Y is None:
            Y = np.zeros((R, w2e.shape[1]), dtype=np.float64)
            U_all = np.zeros((R, de)); H_all = np.zeros((R, de)); dU_all = np.zeros((R, de))
        if hi == lo:
            dW1[e] = np.zeros_like(w1e)
            dW2[e] = np.zeros_like(w2e)
            continue
        g = expert_backward(xp[lo:hi], dYp[lo:hi], w1e, w2e)
        Y[lo:hi] = g["Y"]
        dXp[lo:hi] = g["dX"]
        dW2[e] = g["dW2"]
        dW1[e] = g["dW1"]
        U_all[lo:hi], H_all[lo:hi], dU_all[lo:hi] = g["U"], g["H"], g["dU"]

    # combine backward: gate gradients
    dG = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        dG[:, j] = np.einsum("td,td->t", dy64, Y[inv[:, j]])
    # dispatch backward
    dx = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        dx += dXp[inv[:, j]]
    # router backward through the softmax over all E
    dp = np.zeros((T, E), dtype=np.float64)
    for j in range(k):
        np.add.at(dp, (np.arange(T), idx[:, j].astype(np.int64)), dG[:, j])
    s = (p * dp).sum(axis=1, keepdims=True)
    dlogit = p * (dp - s)
    dx_router = dlogit @ wr64.T
    dx = dx + dx_router
    dWr = x64.T @ dlogit
    dbias = dlogit.sum(axis=0)
    counts = pm["counts"].astype(np.float64)
    return {
        "dx": dx, "dw_router": dWr, "dbias": dbias,
        "dW1": np.stack([dW1[e] for e in range(E)]), "dW2": np.stack([dW2[e] for e in range(E)]),
        "load_frac": counts / R, "mean_prob": p.mean(axis=0),
        # intermediates
        "p": p, "gate": gate, "dG": dG, "dlogit": dlogit, "dYp": dYp, "dXp": dXp, "Y": Y,
        "U": U_all, "H": H_all, "dU": dU_all, "dx_router": dx_router,
        "idx": idx, "counts": pm["counts"], "offsets": offsets, "perm": pm["perm"], "inv": pm["inv"],
    }


def backward(x: np.ndarray, w_router: np.ndarray, router_bias: Optional[np.ndarray], W1: WeightSource,
             W2: WeightSource, k: int, dtype: str, dy: np.ndarray) -> Dict[str, np.ndarray]:
    """The backward of the layer as run: raw workload arrays (bf16 as uint16
    bits), routing on the float32 logits exactly as the forward oracle does it."""
    x64 = decode(x, dtype)
    wr64 = decode(w_router, dtype)
    dy64 = decode(dy, dtype)
    r = route(x64, wr64, router_bias, k)
    w1 = (lambda e: decode(_slice(W1, e), dtype))
    w2 = (lambda e: decode(_slice(W2, e), dtype))
    out = backward64(x64, wr64, w1, w2, k, dy64, r["idx"], r["logits"])
    out["logits"] = r["logits"]
    out["near_tie"] = r["near_tie"]
    return out


def forward64_fixed(x64: np.ndarray, wr64: np.ndarray, bias64: Optional[np.ndarray], W1_64: np.ndarray,
                    W2_64: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """The smooth function the backward differentiates: the forward in float64
    with unrounded logits and the expert choice `idx` held fixed."""
    logits = router_logits(x64, wr64, bias64, rounded=False)
    p = softmax_probs(logits)
    T, k = idx.shape
    y = np.zeros((T, W2_64.shape[2]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            y[t] += p[t, e] * (gelu_tanh(x64[t:t + 1] @ W1_64[e]) @ W2_64[e])[0]
    return y
