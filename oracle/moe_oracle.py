"""Plain, slow CPU oracle of the sparse MoE layer forward (NumPy, float64).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What it computes, and where each step comes from:
  * "Distributed training part 4" (jesamkim's AI tech blog), section 3
    "Mixture of Experts", subsection on structure: the router (gating network)
    is a Linear layer followed by a Softmax that gives each expert a
    probability; the experts are independent FFNs; the output is the sum over
    the top-k experts of the router weight G(x)_i times the expert output
    E_i(x); only the k best experts are selected.
  * same page, section 4 "Expert Parallelism", dispatch/combine: each token is
    sent to the expert it chose and the expert results come back to the token.
    With every expert on one device the exchange is a local permutation:
    rows grouped by expert (dispatch), then gathered back per token (combine).
  * the MOSAIC summary ("Compute-Optimal Is Not Cluster-Optimal", gist.science,
    method item 1) fixes granularity G = d_ff / d_expert, which only sets
    shapes here.

Readings where the pages are silent (each is listed in the design notes):
  * softmax runs over all E logits; the gate of a selected expert is its
    softmax probability, not renormalised over the k selected;
  * selection is made on the float32-rounded logits: descending logit, ties to
    the lower expert index, output order = selection order;
  * an expert is E_i(x) = GELU_tanh(x W1_i) W2_i with no biases, where
    GELU_tanh(u) = u/2 (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)));
  * an optional float32 router bias is added to the logits before both the
    softmax and the selection;
  * no capacity limit: every token gets exactly k experts; groups are ragged
    and may be empty.

Every floating-point step is float64 from the exact input values; routing is a
discrete function of the float32 logits. There is no blocking or fusion: each
step is the definition written out.
"""

from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence, Union

import numpy as np

ArrayLike = Union[np.ndarray, Sequence]


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------

def decode(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact float64 value of a workload tensor.

    bf16 tensors arrive as their raw 16-bit patterns (uint16); a bf16 value is
    the float32 whose upper 16 bits are those bits and whose lower 16 bits are 0.
    """
    if a is None:
        return None
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 tensors are passed as uint16 bit patterns")
        f32 = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f32.astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# router: Linear + Softmax, top-k (blog section 3, structure)
# ---------------------------------------------------------------------------

def router_logits(x64: np.ndarray, wr64: np.ndarray, bias: Optional[np.ndarray],
                  rounded: bool = True) -> np.ndarray:
    """Router Linear: logits = x Wr (+ b), computed in float64 then rounded to float32.

    x64 [T,d], wr64 [d,E] float64; bias [E] float32 or None. Routing is defined
    on the float32 result. With rounded=False the float64 logits are returned
    (and a float64 bias is taken as is): the smooth function whose derivative
    the backward computes.
    """
    logits64 = x64 @ wr64
    if bias is not None:
        b = np.asarray(bias, dtype=np.float32) if rounded else np.asarray(bias, dtype=np.float64)
        logits64 = logits64 + b.astype(np.float64)[None, :]
    return logits64.astype(np.float32) if rounded else logits64


def topk_select(logits32: np.ndarray, k: int) -> np.ndarray:
    """The k best experts per token: sort experts by (-logit, expert index), keep the first k.

    Returns idx [T,k] int32 in selection order (descending logit, ties to the
    lower index). -0.0 and +0.0 compare equal.
    """
    T, E = logits32.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.empty((T, k), dtype=np.int32)
    experts = np.arange(E)
    for t in range(T):
        neg = -logits32[t].astype(np.float64)
        order = np.lexsort((experts, neg))  # primary key: -logit; secondary: index
        idx[t] = order[:k]
    return idx


def softmax_probs(logits: np.ndarray) -> np.ndarray:
    """Softmax over all E logits of each token (float64, max subtracted)."""
    l64 = logits.astype(np.float64)
    m = l64.max(axis=1, keepdims=True)
    ex = np.exp(l64 - m)
    return ex / ex.sum(axis=1, keepdims=True)


def softmax_gates(logits32: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over all E logits (float64, max subtracted); gate = probability of each selected expert."""
    return np.take_along_axis(softmax_probs(logits32), idx.astype(np.int64), axis=1)


def near_ties(logits32: np.ndarray, k: int, margin: float = 1e-6) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest float32 logits differ by less than `margin`.

    For such tokens a different (but equally valid) summation order of the
    router Linear may flip the selection. With k = E there are none.
    """
    T, E = logits32.shape
    if k >= E:
        return np.zeros(T, dtype=bool)
    s = -np.sort(-logits32.astype(np.float64), axis=1)
    return (s[:, k - 1] - s[:, k]) < margin


def route(x64: np.ndarray, wr64: np.ndarray, bias: Optional[np.ndarray], k: int) -> Dict[str, np.ndarray]:
    logits32 = router_logits(x64, wr64, bias)
    idx = topk_select(logits32, k)
    gate = softmax_gates(logits32, idx)
    return {"logits": logits32, "idx": idx, "gate": gate, "near_tie": near_ties(logits32, k)}


# ---------------------------------------------------------------------------
# dispatch as a local permutation (blog section 4, dispatch)
# ---------------------------------------------------------------------------

def permute(idx: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """Group the T*k selections by expert.

    counts[e] = number of (t, j) with idx[t,j] == e; offsets = exclusive prefix
    sum with offsets[E] = T*k. Rows of expert e are its selecting tokens in
    token order: perm[r] = t for row r, and inv[t*k + j] = row of selection (t, j).
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    token_of = np.repeat(np.arange(T, dtype=np.int64), k)
    order = np.lexsort((token_of, flat))  # by expert, then by token
    perm = token_of[order].astype(np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    inv[order] = np.arange(T * k, dtype=np.int32)
    return {"counts": counts, "offsets": offsets, "perm": perm, "inv": inv}


def gather_rows(x64: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Dispatched activations: row r is the input row of token perm[r]."""
    return x64[perm.astype(np.int64)]


# ---------------------------------------------------------------------------
# experts (blog section 3: independent FFNs)
# ---------------------------------------------------------------------------

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """Tanh-form GELU: u/2 * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3))), float64."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(_SQRT_2_OVER_PI * (u + 0.044715 * u * u * u)))


def expert_ffn(X: np.ndarray, w1e: np.ndarray, w2e: np.ndarray) -> np.ndarray:
    """E_i(X) = GELU_tanh(X W1_i) W2_i for the rows of X (float64)."""
    return gelu_tanh(X @ w1e) @ w2e


WeightSource = Union[np.ndarray, Callable[[int], np.ndarray]]


def _slice(W: WeightSource, e: int) -> np.ndarray:
    return W(e) if callable(W) else W[e]


def grouped_ffn(x_perm64: np.ndarray, offsets: np.ndarray, W1: WeightSource, W2: WeightSource) -> np.ndarray:
    """Each expert's FFN on its own contiguous row group [offsets[e], offsets[e+1]).

    W1/W2 are float64 arrays [E,...] or callables e -> float64 slice. Empty
    groups are skipped.
    """
    E = len(offsets) - 1
    R = x_perm64.shape[0]
    d_out = None
    Y = None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w1e, w2e = _slice(W1, e), _slice(W2, e)
        if Y is None:
            d_out = w2e.shape[1]
            Y = np.zeros((R, d_out), dtype=np.float64)
        Y[lo:hi] = expert_ffn(x_perm64[lo:hi], w1e, w2e)
    if Y is None:
        raise ValueError("no rows")
    return Y


# ---------------------------------------------------------------------------
# combine (blog section 3 output formula; section 4 combine)
# ---------------------------------------------------------------------------

def combine(Y_perm: np.ndarray, inv: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """y[t] = sum over j < k of gate[t,j] * Y_perm[inv[t*k+j]], summed in selection order."""
    T, k = gate.shape
    y = np.zeros((T, Y_perm.shape[1]), dtype=np.float64)
    inv2 = inv.reshape(T, k).astype(np.int64)
    for j in range(k):
        y += gate[:, j:j + 1].astype(np.float64) * Y_perm[inv2[:, j]]
    return y


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def forward(x: np.ndarray, w_router: np.ndarray, router_bias: Optional[np.ndarray],
            W1: WeightSource, W2: WeightSource, k: int, dtype: str) -> Dict[str, np.ndarray]:
    """The layer forward: route, dispatch, experts, combine. Inputs are raw workload arrays.

    W1/W2 may also be callables e -> raw slice (decoded here), so large weight
    sets can be streamed one expert at a time.
    """
    x64 = decode(x, dtype)
    wr64 = decode(w_router, dtype)
    E = wr64.shape[1]
    r = route(x64, wr64, router_bias, k)
    p = permute(r["idx"], E)
    xp = gather_rows(x64, p["perm"])
    w1 = (lambda e: decode(_slice(W1, e), dtype))
    w2 = (lambda e: decode(_slice(W2, e), dtype))
    Y_perm = grouped_ffn(xp, p["offsets"], w1, w2)
    y = combine(Y_perm, p["inv"], r["gate"])
    out = dict(r)
    out.update(p)
    out["x_perm"] = xp
    out["Y_perm"] = Y_perm
    out["y"] = y
    return out


def forward_literal(x: np.ndarray, w_router: np.ndarray, router_bias: Optional[np.ndarray],
                    W1: np.ndarray, W2: np.ndarray, k: int, dtype: str) -> np.ndarray:
    """The output formula token by token, with no dispatch: tiny inputs only.

    y[t] = sum over the selected i of G(x_t)_i * E_i(x_t).
    """
    x64 = decode(x, dtype)
    wr64 = decode(w_router, dtype)
    W1_64 = decode(W1, dtype)
    W2_64 = decode(W2, dtype)
    T = x64.shape[0]
    y = np.zeros((T, W2_64.shape[2]), dtype=np.float64)
    for t in range(T):
        logits32 = router_logits(x64[t:t + 1], wr64, router_bias)
        idx = topk_select(logits32, k)[0]
        gate = softmax_gates(logits32, idx[None, :])[0]
        for j in range(k):
            e = int(idx[j])
            y[t] += gate[j] * expert_ffn(x64[t:t + 1], W1_64[e], W2_64[e])[0]
    return y


def forward_tokens(x_rows: np.ndarray, w_router: np.ndarray, router_bias: Optional[np.ndarray],
                   W1_slice: Callable[[int], np.ndarray], W2_slice: Callable[[int], np.ndarray],
                   k: int, dtype: str) -> Dict[str, np.ndarray]:
    """The layer output for a sample of tokens only (their rows of x), one token at a time.

    Each output row depends only on its own token (the FFN and the router are
    token-local), so a sample of rows can be checked without the rest. Weight
    slices are fetched per expert through the callables (raw arrays, decoded here).
    """
    x64 = decode(x_rows, dtype)
    wr64 = decode(w_router, dtype)
    r = route(x64, wr64, router_bias, k)
    T = x64.shape[0]
    # expert outputs per selection, one expert's weights in memory at a time
    per_sel: Dict[tuple, np.ndarray] = {}
    for e in sorted(set(int(v) for v in r["idx"].reshape(-1))):
        w1e, w2e = decode(W1_slice(e), dtype), decode(W2_slice(e), dtype)
        for t in range(T):
            for j in range(k):
                if int(r["idx"][t, j]) == e:
                    per_sel[(t, j)] = expert_ffn(x64[t:t + 1], w1e, w2e)[0]
        del w1e, w2e
    d_out = next(iter(per_sel.values())).shape[0]
    y = np.zeros((T, d_out), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            y[t] += r["gate"][t, j] * per_sel[(t, j)]
    out = dict(r)
    out["y"] = y
    return out
