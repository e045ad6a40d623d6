"""Shared helpers of the GPU parity tests (not collected as tests)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

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
