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

from typing import Dict, Optional

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
                router_zero: bool = False) -> Dict[str, Optional[torch.Tensor]]:
    """Draw x[T,d], w_router[d,E], router_bias[E] (or None), W1[E,d,de], W2[E,de,d].

    All tensors are contiguous, row-major, on `device`, in the workload dtype
    (the bias is float32). With `router_zero` the router weights and bias are
    exact zeros (every logit is then exactly 0).
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
