"""moe_permute_index_noalloc (static device scratch, no workspace argument)
against moe_permute_index (caller workspace) through the C ABI: bit for bit,
on two calls in a row, the second with a smaller problem, so the second call
runs on an array that still holds the first call's contents."""

import pytest
import torch

from gpu_helpers import announce, needs_gpu
from harness import make_routing_table

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run_both(moe, T, E, k, seed):
    idx = make_routing_table(T, E, k, seed=seed, device="cuda", hot=(0,), cold=(E - 1,))
    p = moe.make_problem(T, 128, E, k, 256, torch.bfloat16)
    R = T * k
    dev = idx.device
    ref = {n: torch.full((m,), -7, dtype=torch.int32, device=dev)
           for n, m in (("counts", E), ("offsets", E + 1), ("perm", R), ("inv", R))}
    got = {n: torch.full_like(v, -9) for n, v in ref.items()}
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_STAGE_PERMUTE), dtype=torch.uint8, device=dev)
    moe.moe_permute_index(p, idx, ref["counts"], ref["offsets"], ref["perm"], ref["inv"], ws)
    moe.moe_permute_index_noalloc(p, idx, got["counts"], got["offsets"], got["perm"], got["inv"])
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(got[n], ref[n]), (T, E, k, n)
    assert int(ref["offsets"][-1]) == R


def test_noalloc_permute_matches_workspace_permute(moe):
    # a large problem (separate scan launch: more than 64 blocks of 256 tokens),
    # then a smaller one (scan fused into the scatter) on the same static array,
    # then one small enough for the one-workgroup form (no scratch at all)
    for T, E, k, seed in ((40000, 256, 8, 1), (3000, 16, 4, 2), (700, 8, 2, 3)):
        announce(f"noalloc permute T={T} E={E} k={k}")
        _run_both(moe, T, E, k, seed)
