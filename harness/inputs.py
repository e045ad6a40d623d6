"""Seeded synthetic input tensors for a MoE workload.

Recipe (one per tensor, independent of generation order):
  * every tensor (or expert slice of a weight tensor) gets its own torch
    Philox/MT generator on the target device, seeded by a fixed integer mix of
    (seed, tensor id, slice index);
  * values are float32 standard normals times the configured standard
    deviation, then rounded once to the workload dtype (bf16 round-to-nearest-
    even via torch's conversion, or kept as float32);
  * the router bias, when the workload has one, is an exact float32 vector.

Tensors are drawn on the device that will consume them (the GPU for the GPU
path, the CPU for host-only tests). A CPU check of GPU results receives host
copies of the very tensors the GPU used; nothing here depends on the MoE
arithmetic.
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np
import torch

from .configs import MoEConfig

# tensor ids for seeding
_X, _WR, _W1, _W2 = 1, 2, 3, 4


def _mix(seed: int, tensor: int, slice_: int) -> int:
    """Fixed 63-bit integer mix of the three seeding coordinates (splitmix64 steps)."""
    mask = (1 << 64) - 1
    z = (seed * 0x9E3779B97F4A7C15 + tensor * 0xBF58476D1CE4E5B9 + slice_ * 0x94D049BB133111EB
         + 0x2545F4914F6CDD1D) & mask
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
    z = z ^ (z >> 31)
    return z & ((1 << 63) - 1)


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _normal(shape, std: float, seed: int, tensor: int, slice_: int, device, dtype: torch.dtype,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(seed, tensor, slice_))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v.mul_(float(std))
    if out is None:
        return v.to(dtype)
    out.copy_(v)  # rounds to out.dtype (round-to-nearest-even for bf16)
    return out


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu",
                router_zero: bool = False, weights: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Draw x[T,d], w_router[d,E], router_bias[E] (or None), W1[E,d,de], W2[E,de,d].

    All tensors are contiguous, row-major, on `device`, in the workload dtype
    (the bias is float32). With `router_zero` the router weights and bias are
    exact zeros (every logit is then exactly 0). With `weights=False` the expert
    weights are not drawn (W1 and W2 are None).
    """
    dev = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    x = _normal((cfg.T, cfg.d_model), cfg.x_std, seed, _X, 0, dev, dt)
    if router_zero:
        wr = torch.zeros((cfg.d_model, cfg.E), device=dev, dtype=dt)
    else:
        wr = _normal((cfg.d_model, cfg.E), cfg.router_std, seed, _WR, 0, dev, dt)
    bias = None
    bv = cfg.bias_vector()
    if router_zero:
        bias = torch.zeros(cfg.E, device=dev, dtype=torch.float32) if bv is not None else None
    elif bv is not None:
        bias = torch.tensor(bv, dtype=torch.float32, device=dev)
    if not weights:
        return {"x": x, "w_router": wr, "router_bias": bias, "W1": None, "W2": None}
    W1 = torch.empty((cfg.E, cfg.d_model, cfg.d_expert), device=dev, dtype=dt)
    W2 = torch.empty((cfg.E, cfg.d_expert, cfg.d_model), device=dev, dtype=dt)
    for e in range(cfg.E):
        _normal((cfg.d_model, cfg.d_expert), cfg.w1_std, seed, _W1, e, dev, dt, out=W1[e])
        _normal((cfg.d_expert, cfg.d_model), cfg.w2_std, seed, _W2, e, dev, dt, out=W2[e])
    return {"x": x, "w_router": wr, "router_bias": bias, "W1": W1, "W2": W2}


def host_array(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host copy as numpy: bf16 tensors become their raw uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def to_host_arrays(inputs: Dict[str, Optional[torch.Tensor]]) -> Dict[str, Optional[np.ndarray]]:
    return {k: host_array(v) for k, v in inputs.items()}


def make_exact_router_inputs(cfg: MoEConfig, seed: int = 0, device="cpu", bias: bool = False,
                             tie_group: int = 1):
    """Router inputs whose float32 logits are exact whatever the summation order.

    x takes values in {-3..3}/4 and w_router in {-7..7}/64 (exact in bf16 and
    float32), so every product is a multiple of 2^-8 and every partial sum of a
    row stays below 2^15 in magnitude for d_model <= 2^14: all partial sums are
    exactly representable. Equal logits are frequent, which exercises the
    tie-break. With `bias`, a bias in multiples of 1/8 is added. With
    tie_group = g > 1, experts come in runs of g identical router columns (and
    biases), so every token has exact ties, also at the k-th place.
    """
    dev = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    g = torch.Generator(device="cpu")
    g.manual_seed(_mix(seed, 11, 0))
    x = (torch.randint(-3, 4, (cfg.T, cfg.d_model), generator=g).float() / 4).to(dt).to(dev)
    wr = (torch.randint(-7, 8, (cfg.d_model, cfg.E), generator=g).float() / 64).to(dt).to(dev)
    b = None
    if bias:
        b = (torch.randint(-16, 17, (cfg.E,), generator=g).float() / 8).to(dev)
    if tie_group > 1:
        src = (torch.arange(cfg.E) // tie_group) * tie_group
        wr = wr[:, src.to(dev)].contiguous()
        if b is not None:
            b = b[src.to(dev)].contiguous()
    return {"x": x, "w_router": wr, "router_bias": b}


def make_routing_table(T: int, E: int, k: int, seed: int = 0, device="cpu",
                       hot: Optional[Tuple[int, ...]] = None, cold: Tuple[int, ...] = ()) -> torch.Tensor:
    """A random routing table idx[T,k] int32: k distinct experts per token.

    `hot` experts are chosen by every token (when k allows); `cold` experts are
    never chosen, which leaves their groups empty.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(_mix(seed, 12, T * 1000003 + E * 131 + k))
    allowed = [e for e in range(E) if e not in set(cold)]
    hot = tuple(e for e in (hot or ()) if e in allowed)[:k]
    rest = [e for e in allowed if e not in hot]
    need = k - len(hot)
    if need > len(rest):
        raise ValueError("not enough experts left for k distinct choices")
    scores = torch.rand((T, len(rest)), generator=g)
    pick = torch.argsort(scores, dim=1)[:, :need]
    rest_t = torch.tensor(rest, dtype=torch.int64)
    cols = [torch.full((T, 1), h, dtype=torch.int64) for h in hot] + [rest_t[pick]]
    idx = torch.cat(cols, dim=1)
    # shuffle the order inside each row so hot experts are not always first
    order = torch.argsort(torch.rand((T, k), generator=g), dim=1)
    idx = torch.gather(idx, 1, order)
    return idx.to(torch.int32).to(device)


def make_group_offsets(E: int, rows: int, seed: int = 0, empty: Tuple[int, ...] = ()) -> torch.Tensor:
    """offsets[E+1] (int32, on the CPU) of random ragged group sizes summing to `rows`.

    Experts listed in `empty` get no rows.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(_mix(seed, 13, E * 7919 + rows))
    live = [e for e in range(E) if e not in set(empty)]
    if not live:
        raise ValueError("at least one non-empty group is needed")
    w = torch.rand(len(live), generator=g) + 0.05
    sizes = torch.floor(w / w.sum() * rows).to(torch.int64)
    sizes[0] += rows - int(sizes.sum())
    counts = torch.zeros(E, dtype=torch.int64)
    counts[torch.tensor(live)] = sizes
    off = torch.zeros(E + 1, dtype=torch.int64)
    off[1:] = torch.cumsum(counts, 0)
    return off.to(torch.int32)


def make_dense(shape, std: float, seed: int, tag: int, device="cpu", dtype: str = "bf16") -> torch.Tensor:
    """A seeded normal tensor in the workload dtype (for stage-level parity inputs)."""
    return _normal(tuple(shape), std, seed, 20 + tag, 0, torch.device(device), torch_dtype(dtype))
