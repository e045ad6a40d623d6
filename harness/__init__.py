"""Seeded synthetic inputs for the sparse MoE layer forward.

This package only draws random tensors of the workloads' shapes and
distributions. It holds none of the layer's arithmetic (no router, no top-k,
no expert FFN, no combine), so both the CPU oracle's tests and the GPU path's
tests and benchmark may use it without sharing any of the method's code.
"""

from .configs import CONFIGS, MoEConfig, get_config, scaled_config  # noqa: F401
from .inputs import (  # noqa: F401
    host_array,
    make_dense,
    make_exact_router_inputs,
    make_group_offsets,
    make_inputs,
    make_routing_table,
    to_host_arrays,
)
