"""Shared helpers of the GPU parity tests (not collected as tests)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle

U32 = 2.0 ** -24  # float32 unit roundoff

# Output tolerances: max|y_gpu - y_ref| / max|y_ref|
TOL_BF16 = 1e-2
TOL_F32 = 1e-5

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU visible")


def announce(msg: str):
    """Print what a GPU step is about to run, flushed, so a failing run names its case."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a GPU float tensor (bf16 and float32 widen exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def i64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / den)


def logit_bound(x64: np.ndarray, wr64: np.ndarray, bias, logits_ref: np.ndarray) -> np.ndarray:
    """Rounding bound of a float32 dot product of length d against the exact value.

    |fl(sum) - sum| <= (d + 1) u sum|x w| for any summation order (products of
    bf16 values are exact in float32; float32 products add one rounding, covered
    by the +1), plus the bias addition and the reference's own rounding to float32.
    """
    d = x64.shape[1]
    s = np.abs(x64) @ np.abs(wr64)
    b = 0.0 if bias is None else np.abs(np.asarray(bias, dtype=np.float64))[None, :]
    return (d + 2) * U32 * s + 2 * U32 * (np.abs(logits_ref) + b)


def check_topk_valid(idx: np.ndarray, logits: np.ndarray):
    """idx[t] must be the top-k of the logits row (descending, ties to the lower index).

    A validity check of a result against its own logits: any correct top-k of
    these float32 values gives exactly this sequence.
    """
    T, k = idx.shape
    E = logits.shape[1]
    experts = np.arange(E)
    for t in range(T):
        order = np.lexsort((experts, -logits[t].astype(np.float64)))[:k]
        if not np.array_equal(order, idx[t]):
            raise AssertionError(f"token {t}: idx {idx[t].tolist()} is not the top-{k} {order.tolist()} "
                                 f"of its logits")


def check_routing_exact(cfg, st):
    """R-exact: idx is the top-k of the GPU's own logits, and counts, offsets,
    perm and inv are the oracle's dispatch of that idx, bit for bit."""
    logits = f64(st["logits"]).astype(np.float32)
    idx = i64(st["idx"])
    check_topk_valid(idx, logits)
    pm = oracle.permute(idx, cfg.E)
    for key in ("counts", "offsets", "perm", "inv"):
        got = i64(st[key])
        if not np.array_equal(got, pm[key]):
            bad = np.nonzero(got != pm[key])[0]
            raise AssertionError(f"{cfg.name}: {key} differs from the oracle's dispatch of the GPU's idx at "
                                 f"{bad.size} positions, first {bad[:5].tolist()}")
    return logits, idx, pm


def check_routing_e2e(cfg, logits, idx, gate, x64, wr64, bias, ref):
    """R-logits and R-e2e against the oracle's own routing; returns the mask of
    tokens kept for the output comparison (outside near-ties)."""
    dl = np.abs(logits.astype(np.float64) - ref["logits"].astype(np.float64))
    bound = logit_bound(x64, wr64, bias, ref["logits"])
    assert np.all(dl <= bound), f"{cfg.name}: logit error {dl.max():.3e} above the float32 bound"
    tie = ref["near_tie"]
    same = np.sort(idx, axis=1) == np.sort(ref["idx"].astype(np.int64), axis=1)
    same = same.all(axis=1)
    bad = np.nonzero(~same & ~tie)[0]
    assert bad.size == 0, f"{cfg.name}: {bad.size} tokens route differently outside near-ties, e.g. {bad[:5]}"
    ok = same & ~tie
    # gates of the tokens with the same set: the bound implied by the logit difference
    order_g = np.argsort(idx[ok], axis=1)
    order_r = np.argsort(ref["idx"][ok].astype(np.int64), axis=1)
    g_gpu = np.take_along_axis(gate[ok], order_g, axis=1)
    g_ref = np.take_along_axis(ref["gate"][ok], order_r, axis=1)
    rel = np.abs(g_gpu - g_ref) / g_ref
    gtol = 2 * dl[ok].max(axis=1, keepdims=True) + 32 * U32
    assert np.all(rel <= gtol), f"{cfg.name}: gate error {rel.max():.3e}"
    print(f"{cfg.name}: max|dlogit| {dl.max():.3e}, near-ties {int(tie.sum())} "
          f"(routed differently {int((~same).sum())})", flush=True)
    return ~tie
