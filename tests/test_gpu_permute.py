"""moe_permute on the GPU: counts, offsets, perm, inv and x_perm are integer and
copy results, so they must equal the oracle's bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import announce, i64, needs_gpu
from harness import host_array, make_dense, make_routing_table

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_permute(moe, T, d, E, k, dtype, idx, x):
    p = moe.make_problem(T, d, E, k, 64, dtype)
    dev = idx.device
    R = T * k
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    perm = torch.full((R,), -7, dtype=torch.int32, device=dev)
    inv = torch.full((R,), -7, dtype=torch.int32, device=dev)
    x_perm = torch.zeros((R, d), dtype=x.dtype, device=dev)
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_PERMUTE), dtype=torch.uint8, device=dev)
    moe.moe_permute(p, idx, x, counts, offsets, perm, inv, x_perm, ws)
    torch.cuda.synchronize()
    return counts, offsets, perm, inv, x_perm


CASES = [
    # T, d, E, k, dtype, hot, cold
    (1, 64, 1, 1, "bf16", (), ()),
    (5, 64, 8, 2, "f32", (), ()),
    (255, 128, 8, 2, "bf16", (), ()),
    (256, 128, 8, 2, "bf16", (), ()),
    (257, 128, 8, 2, "bf16", (), ()),
    (1000, 256, 64, 8, "bf16", (0, 1), (60, 61, 62, 63)),
    (4096, 2048, 8, 2, "bf16", (), ()),
    (3001, 128, 256, 8, "bf16", (), tuple(range(100, 140))),
    (700, 64, 16, 16, "f32", (), ()),
    (300, 64, 256, 256, "bf16", (), ()),
    # batches of at most 1024 tokens with k <= 8 run in one workgroup: its limits
    (1024, 64, 256, 8, "bf16", (5,), tuple(range(200, 256))),
    (1025, 64, 256, 8, "bf16", (5,), ()),
    (64, 64, 8, 1, "bf16", (), (7,)),
    # the scan stages per-block counts in LDS in chunks of 16384: several chunks,
    # E not a power of two, and k above 8 (selections handled in groups of 8)
    (40000, 64, 256, 8, "bf16", (3,), tuple(range(10, 30))),
    (70000, 64, 200, 3, "f32", (), ()),
    (20000, 64, 64, 12, "bf16", (), (0,)),
]


@pytest.mark.parametrize("T,d,E,k,dtype,hot,cold", CASES)
def test_permute_bit_exact(moe, T, d, E, k, dtype, hot, cold):
    announce(f"permute T={T} d={d} E={E} k={k} {dtype} hot={hot} cold={len(cold)}")
    idx = make_routing_table(T, E, k, seed=3, device="cuda", hot=hot, cold=cold)
    x = make_dense((T, d), 1.0, seed=3, tag=1, device="cuda", dtype=dtype)
    counts, offsets, perm, inv, x_perm = run_permute(moe, T, d, E, k, dtype, idx, x)
    ref = oracle.permute(i64(idx).astype(np.int32), E)
    assert np.array_equal(i64(counts), ref["counts"])
    assert np.array_equal(i64(offsets), ref["offsets"])
    assert np.array_equal(i64(perm), ref["perm"])
    assert np.array_equal(i64(inv), ref["inv"])
    xh = host_array(x)
    assert np.array_equal(host_array(x_perm), xh[ref["perm"]])
    for e in cold:
        assert ref["counts"][e] == 0


def test_permute_skewed_full_size(moe):
    """The skewed workload's shape: 16384 tokens, 64 experts, top-8, two experts
    chosen by every token and four never chosen."""
    T, d, E, k = 16384, 2048, 64, 8
    announce("permute skewed full size")
    idx = make_routing_table(T, E, k, seed=4, device="cuda", hot=(0, 1), cold=(60, 61, 62, 63))
    x = make_dense((T, d), 1.0, seed=4, tag=1, device="cuda")
    counts, offsets, perm, inv, x_perm = run_permute(moe, T, d, E, k, "bf16", idx, x)
    ref = oracle.permute(i64(idx).astype(np.int32), E)
    assert np.array_equal(i64(offsets), ref["offsets"])
    assert np.array_equal(i64(perm), ref["perm"])
    assert np.array_equal(i64(inv), ref["inv"])
    rows = np.random.default_rng(0).choice(T * k, 4096, replace=False)
    assert np.array_equal(host_array(x_perm[torch.from_numpy(rows).cuda()]), host_array(x)[ref["perm"][rows]])


def test_permute_ignores_out_of_range_experts(moe):
    """Entries outside [0, E) select nothing: inv is -1 for them and the rest is
    the permutation of the valid selections."""
    T, d, E, k = 300, 64, 8, 2
    announce("permute out-of-range entries")
    idx = make_routing_table(T, E, k, seed=5, device="cuda")
    bad = torch.tensor([[3, 0], [17, 1], [250, 1]])
    for t, j in bad[:, :2].tolist():
        idx[t, j] = -1 if t == 3 else 99
    x = make_dense((T, d), 1.0, seed=5, tag=1, device="cuda")
    counts, offsets, perm, inv, x_perm = run_permute(moe, T, d, E, k, "bf16", idx, x)
    ih = i64(idx)
    valid = (ih >= 0) & (ih < E)
    assert int(i64(offsets)[E]) == int(valid.sum())
    invh = i64(inv).reshape(T, k)
    assert np.all(invh[~valid] == -1)
    ph = i64(perm)
    for t, j in zip(*np.nonzero(valid)):
        assert ph[invh[t, j]] == t


@pytest.mark.parametrize("T,E,k", [(1025, 256, 8), (5000, 64, 8), (16384, 8, 2), (9999, 200, 3)])
def test_permute_scan_inside_scatter(moe, T, E, k):
    """Up to 64 blocks of tokens the scatter blocks run the scan themselves
    (no scan launch); forced back to the separate scan (MOE_PERMUTE_FUSED_SCAN=0)
    every output is the same, bit for bit, and equals the oracle's."""
    import os
    announce(f"permute fused scan T={T} E={E} k={k}")
    idx = make_routing_table(T, E, k, seed=21, hot=(1,)).cuda()
    x = make_dense((T, 64), 1.0, seed=21, tag=1, device="cuda", dtype="bf16")
    fused = run_permute(moe, T, 64, E, k, "bf16", idx, x)
    os.environ["MOE_PERMUTE_FUSED_SCAN"] = "0"
    try:
        split = run_permute(moe, T, 64, E, k, "bf16", idx, x)
    finally:
        del os.environ["MOE_PERMUTE_FUSED_SCAN"]
    for a, b in zip(fused, split):
        assert torch.equal(a, b)
    ref = oracle.permute(i64(idx).astype(np.int32), E)
    for name, got in zip(("counts", "offsets", "perm", "inv"), fused[:4]):
        assert np.array_equal(i64(got), ref[name]), name
