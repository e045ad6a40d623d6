"""Workload registry: the five layer shapes the MoE forward is tested and measured on.

Shapes follow the MoE layer of "Distributed training part 4" (jesamkim's AI
tech blog, section 3 "Mixture of Experts"): a router over E experts, top-k
selection (k = 1 or 2 typically; 8 for fine-grained layers), and E independent
FFN experts. The granularity G = d_ff / d_expert comes from the MOSAIC summary
("Compute-Optimal Is Not Cluster-Optimal", gist.science, method item 1): the
fine-grained workloads split a d_ff = 8192 FFN into G = 8 experts of 1024.

Init reading: a bare decimal such as 0.02 is a standard deviation; a fan-in
fraction 1/n is a variance, so the standard deviation is n ** -0.5.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d_model: int
    E: int
    k: int
    d_expert: int
    dtype: str  # "f32" or "bf16"
    x_std: float
    router_std: float
    w1_std: float
    w2_std: float
    # (expert index, additive router-logit bias); None means no bias vector
    router_bias: Optional[Tuple[Tuple[int, float], ...]] = None
    description: str = ""

    @property
    def rows(self) -> int:
        """Total (token, expert) selections, i.e. rows of the permuted buffers."""
        return self.T * self.k

    def ffn_flops(self) -> int:
        """Algorithmic FLOPs of the two expert GEMMs: 2 MACs-as-flops each."""
        return 4 * self.T * self.k * self.d_model * self.d_expert

    def router_flops(self) -> int:
        return 2 * self.T * self.d_model * self.E

    def bias_vector(self):
        if self.router_bias is None:
            return None
        b = [0.0] * self.E
        for e, v in self.router_bias:
            b[e] = float(v)
        return b

    def describe(self) -> Dict[str, object]:
        return {
            "workload": self.name,
            "T": self.T,
            "d_model": self.d_model,
            "E": self.E,
            "k": self.k,
            "d_expert": self.d_expert,
            "dtype": self.dtype,
            "router_bias": self.router_bias is not None,
        }


def _cfgs():
    c = {}
    c["tiny_fp32"] = MoEConfig(
        "tiny_fp32", T=64, d_model=128, E=8, k=2, d_expert=256, dtype="f32",
        x_std=1.0, router_std=0.02, w1_std=128 ** -0.5, w2_std=256 ** -0.5,
        description="T=64 d=128 E=8 top-2 d_expert=256, fp32")
    c["mixtral_coarse"] = MoEConfig(
        "mixtral_coarse", T=4096, d_model=2048, E=8, k=2, d_expert=8192, dtype="bf16",
        x_std=1.0, router_std=0.02, w1_std=2048 ** -0.5, w2_std=8192 ** -0.5,
        description="T=4096 d=2048 E=8 top-2 d_expert=8192 (G=1), bf16")
    c["fine_grained"] = MoEConfig(
        "fine_grained", T=8192, d_model=2048, E=64, k=8, d_expert=1024, dtype="bf16",
        x_std=1.0, router_std=0.02, w1_std=2048 ** -0.5, w2_std=1024 ** -0.5,
        description="T=8192 d=2048 E=64 top-8 d_expert=1024 (G=8), bf16")
    c["skewed"] = MoEConfig(
        "skewed", T=16384, d_model=2048, E=64, k=8, d_expert=1024, dtype="bf16",
        x_std=1.0, router_std=0.02, w1_std=2048 ** -0.5, w2_std=1024 ** -0.5,
        router_bias=((0, 3.0), (1, 3.0), (60, -6.0), (61, -6.0), (62, -6.0), (63, -6.0)),
        description="T=16384 d=2048 E=64 top-8 d_expert=1024, bf16, router bias "
                    "+3 on experts 0,1 and -6 on 60..63")
    c["large_sparse"] = MoEConfig(
        "large_sparse", T=16384, d_model=7168, E=256, k=8, d_expert=2048, dtype="bf16",
        x_std=1.0, router_std=0.006, w1_std=7168 ** -0.5, w2_std=2048 ** -0.5,
        description="T=16384 d=7168 E=256 top-8 d_expert=2048, bf16 (~15 GB experts)")
    return c


CONFIGS: Dict[str, MoEConfig] = _cfgs()
CONFIG_ORDER = ("tiny_fp32", "mixtral_coarse", "fine_grained", "skewed", "large_sparse")


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]


def scaled_config(name: str, T: Optional[int] = None, d_model: Optional[int] = None,
                  E: Optional[int] = None, k: Optional[int] = None,
                  d_expert: Optional[int] = None, dtype: Optional[str] = None,
                  suffix: str = "small") -> MoEConfig:
    """A smaller workload with the same distributions, for oracle-sized parity runs.

    The weight standard deviations keep their fan-in reading for the new sizes.
    A router bias that names experts beyond the new E is dropped for those experts.
    """
    base = CONFIGS[name]
    T = base.T if T is None else T
    d_model = base.d_model if d_model is None else d_model
    E = base.E if E is None else E
    k = base.k if k is None else k
    d_expert = base.d_expert if d_expert is None else d_expert
    bias = None
    if base.router_bias is not None:
        kept = tuple((e, v) for e, v in base.router_bias if e < E)
        if E >= 6 and base.name == "skewed":
            # keep the pattern's shape: two favoured experts, the last four disfavoured
            kept = ((0, 3.0), (1, 3.0)) + tuple((E - 4 + i, -6.0) for i in range(4))
        bias = kept or None
    return dataclasses.replace(
        base, name=f"{base.name}_{suffix}", T=T, d_model=d_model, E=E, k=k,
        d_expert=d_expert, dtype=dtype or base.dtype,
        w1_std=d_model ** -0.5, w2_std=d_expert ** -0.5, router_bias=bias)


def fan_in_std(n: int) -> float:
    return 1.0 / math.sqrt(n)
