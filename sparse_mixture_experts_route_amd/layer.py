"""Convenience wrapper: buffers for one layer shape, allocated once with torch.

torch only provides device memory here; the forward itself is the library's
moe_forward (or the four stage entry points) on the current HIP stream.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib


class MoEForward:
    """Holds outputs and workspace for a fixed (T, d_model, E, k, d_expert, dtype)."""

    def __init__(self, T: int, d_model: int, E: int, k: int, d_expert: int, dtype: torch.dtype,
                 device="cuda"):
        self.problem = _lib.make_problem(T, d_model, E, k, d_expert, dtype)
        self.dtype = dtype
        self.device = torch.device(device)
        ws_bytes = _lib.moe_workspace_size(self.problem, _lib.MOE_STAGE_FORWARD)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        self.y = torch.empty((T, d_model), dtype=dtype, device=self.device)

    def __call__(self, x: torch.Tensor, w_router: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor,
                 router_bias: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        _lib.moe_forward(self.problem, x, w_router, router_bias, W1, W2, self.y, self.ws, stream)
        return self.y

    def stages(self, x, w_router, W1, W2, router_bias=None, stream=None, logits=True):
        """Run the four stage entry points one after another; return every intermediate.

        Routing goes through moe_route_ws, the router moe_forward runs, so both
        paths select on logits summed in the same order."""
        p = self.problem
        T, E, k = p.T, p.E, p.k
        R = T * k
        dev = self.device
        out = {
            "logits": torch.empty((T, E), dtype=torch.float32, device=dev) if logits else None,
            "idx": torch.empty((T, k), dtype=torch.int32, device=dev),
            "gate": torch.empty((T, k), dtype=torch.float32, device=dev),
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "perm": torch.empty(R, dtype=torch.int32, device=dev),
            "inv": torch.empty(R, dtype=torch.int32, device=dev),
            "x_perm": torch.empty((R, p.d_model), dtype=self.dtype, device=dev),
            "y_perm": torch.empty((R, p.d_model), dtype=self.dtype, device=dev),
            "y": torch.empty((T, p.d_model), dtype=self.dtype, device=dev),
        }
        ws_p = torch.empty(_lib.moe_workspace_size(p, _lib.MOE_STAGE_PERMUTE), dtype=torch.uint8, device=dev)
        ws_f = torch.empty(_lib.moe_workspace_size(p, _lib.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device=dev)
        ws_r = torch.empty(_lib.moe_workspace_size(p, _lib.MOE_STAGE_ROUTE), dtype=torch.uint8, device=dev)
        _lib.moe_route_ws(p, x, w_router, router_bias, out["logits"], out["idx"], out["gate"], ws_r, stream)
        _lib.moe_permute(p, out["idx"], x, out["counts"], out["offsets"], out["perm"], out["inv"], out["x_perm"],
                         ws_p, stream)
        _lib.moe_grouped_ffn(p, out["x_perm"], out["offsets"], W1, W2, out["y_perm"], ws_f, stream)
        _lib.moe_combine(p, out["y_perm"], out["inv"], out["gate"], out["y"], stream)
        return out
