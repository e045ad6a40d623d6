"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

Thin Python binding over libmoe.so's C ABI (include/moe.h): the functions
below carry the C names and only marshal arguments (torch tensors are device
buffers; their data pointers and torch's current HIP stream go to the
library). Every step of the layer runs in the library's HIP kernels; there is
no CPU or PyTorch fallback, and importing fails when the library is missing.
"""

from ._lib import (  # noqa: F401
    MOE_DTYPE_BF16,
    MOE_DTYPE_F32,
    MOE_STAGE_FORWARD,
    MOE_STAGE_GROUPED_FFN,
    MOE_STAGE_PERMUTE,
    MOE_STAGE_ROUTE,
    MOE_STAGE_TRAIN,
    MoEError,
    Problem,
    lib_path,
    make_problem,
    moe_combine,
    moe_backward,
    moe_forward,
    moe_forward_train,
    moe_grouped_ffn,
    moe_grouped_ffn_gather,
    moe_permute,
    moe_permute_index,
    moe_permute_index_noalloc,
    moe_plan,
    moe_route,
    moe_route_ws,
    moe_status_str,
    moe_workspace_size,
)
from .layer import MoEForward  # noqa: F401
