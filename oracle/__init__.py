"""CPU oracle for the sparse MoE layer forward and backward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python binding)
never calls it and never falls back to it.
"""

from .moe_oracle import (  # noqa: F401
    decode,
    router_logits,
    topk_select,
    softmax_gates,
    near_ties,
    route,
    permute,
    gather_rows,
    gelu_tanh,
    expert_ffn,
    grouped_ffn,
    combine,
    forward,
    forward_literal,
    forward_tokens,
    softmax_probs,
)
from .moe_backward import (  # noqa: F401
    backward,
    backward64,
    expert_backward,
    forward64_fixed,
    gelu_tanh_grad,
)
