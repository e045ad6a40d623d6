"""moe_combine on the GPU against the oracle's gate-weighted gather."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import U32, announce, f64, i64, needs_gpu, rel_err
from harness import make_dense, make_routing_table

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("T,d,E,k,dtype", [
    (1, 64, 4, 1, "bf16"), (64, 128, 8, 2, "f32"), (333, 2048, 8, 2, "bf16"),
    (1000, 256, 64, 8, "bf16"), (257, 7168, 256, 8, "bf16"), (50, 64, 16, 16, "f32"),
])
def test_combine_against_oracle(moe, T, d, E, k, dtype):
    announce(f"combine T={T} d={d} k={k} {dtype}")
    R = T * k
    idx = make_routing_table(T, E, k, seed=9)
    ref_p = oracle.permute(idx.numpy(), E)  # a genuine inverse permutation of some routing
    inv = torch.from_numpy(ref_p["inv"]).cuda()
    y_perm = make_dense((R, d), 1.0, seed=9, tag=1, device="cuda", dtype=dtype)
    g = torch.Generator().manual_seed(T)
    gate = torch.rand((T, k), generator=g).cuda()
    p = moe.make_problem(T, d, E, k, 64, dtype)
    y = torch.empty((T, d), dtype=y_perm.dtype, device="cuda")
    moe.moe_combine(p, y_perm, inv, gate, y)
    torch.cuda.synchronize()
    ref = oracle.combine(f64(y_perm), i64(inv).astype(np.int32), f64(gate))
    err = rel_err(f64(y), ref)
    # bf16: one rounding of the float32 sum (2^-9 relative) plus float32 accumulation
    tol = 2 ** -8 if dtype == "bf16" else 4 * k * U32 * 4
    print(f"combine {dtype} T={T} k={k}: rel err {err:.3e} (tol {tol:.1e})")
    assert err <= tol


def test_combine_skips_ignored_selections(moe):
    """inv entries of -1 (selections the permute ignored) contribute nothing."""
    T, d, E, k = 10, 64, 4, 2
    announce("combine ignored selections")
    y_perm = make_dense((T * k, d), 1.0, seed=10, tag=1, device="cuda", dtype="f32")
    inv = torch.arange(T * k, dtype=torch.int32, device="cuda")
    inv[1::2] = -1
    gate = torch.full((T, k), 0.5, device="cuda")
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(moe.make_problem(T, d, E, k, 64, "f32"), y_perm, inv, gate, y)
    torch.cuda.synchronize()
    assert torch.equal(y, 0.5 * y_perm[0::2])


@pytest.mark.parametrize("T,d,k", [(333, 2048, 2), (1000, 256, 8), (257, 7168, 8), (40, 1088, 12)])
def test_combine_streaming_accesses_match(moe, T, d, k):
    """The non-temporal variant (chosen for large y_perm) and the plain one do
    the same arithmetic: bit-equal outputs, and the oracle's within tolerance."""
    import os
    E = 64
    announce(f"combine streaming T={T} d={d} k={k}")
    idx = make_routing_table(T, E, k, seed=11)
    inv = torch.from_numpy(oracle.permute(idx.numpy(), E)["inv"]).cuda()
    y_perm = make_dense((T * k, d), 1.0, seed=11, tag=1, device="cuda", dtype="bf16")
    gate = torch.rand((T, k), generator=torch.Generator().manual_seed(11)).cuda()
    p = moe.make_problem(T, d, E, k, 64, "bf16")
    out = []
    for nt in ("0", "1"):
        os.environ["MOE_COMBINE_NT"] = nt
        try:
            y = torch.full((T, d), float("nan"), dtype=y_perm.dtype, device="cuda")
            moe.moe_combine(p, y_perm, inv, gate, y)
            torch.cuda.synchronize()
        finally:
            del os.environ["MOE_COMBINE_NT"]
        out.append(y)
    assert torch.equal(out[0], out[1])
    ref = oracle.combine(f64(y_perm), i64(inv).astype(np.int32), f64(gate))
    assert rel_err(f64(out[1]), ref) <= 2 ** -8
