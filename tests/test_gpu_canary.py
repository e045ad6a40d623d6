"""Every entry point writes its outputs and workspace only, and never its inputs.

Each output and each workspace sits inside a larger allocation whose 64 KiB
bands before and after it hold a known byte pattern (the "canary"). After the
call and a synchronisation the bands must be unchanged. Every input must
also be bit for bit what it was. The shapes are ragged (no width or row count
a multiple of a tile), decode-sized (the split router and 32-row tile), float32,
and a training step (moe_forward_train and moe_backward sharing one workspace).
"""

import math

import pytest
import torch

from gpu_helpers import announce, needs_gpu
from harness import make_dense, make_inputs, scaled_config

pytestmark = [pytest.mark.gpu, needs_gpu]

BAND = 1 << 16
CANARY = 0xA5


class Guarded:
    """A tensor of `shape` and `dtype` inside a canary-banded byte buffer."""

    def __init__(self, shape, dtype):
        self.nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        span = (self.nbytes + 255) // 256 * 256
        self.buf = torch.full((BAND + span + BAND,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[BAND:BAND + self.nbytes].view(dtype).view(shape)

    def intact(self) -> bool:
        return bool((self.buf[:BAND] == CANARY).all()) and bool((self.buf[BAND + self.nbytes:] == CANARY).all())


def ws_guard(moe, p, stage):
    return Guarded((moe.moe_workspace_size(p, stage),), torch.uint8)


def check(name, guards, inputs, before):
    torch.cuda.synchronize()
    for gname, g in guards.items():
        assert g.intact(), f"{name}: wrote outside {gname}"
    for iname, t in inputs.items():
        assert torch.equal(t, before[iname]), f"{name}: changed its input {iname}"


CASES = [
    # name, T, d_model, E, k, d_expert, dtype
    ("ragged", 777, 320, 12, 3, 448, "bf16"),
    ("decode", 5, 512, 16, 2, 1024, "bf16"),
    ("decode_mid", 40, 768, 24, 2, 576, "bf16"),
    ("fp32", 70, 128, 8, 2, 256, "f32"),
]


@pytest.mark.parametrize("name,T,d,E,k,de,dtype", CASES, ids=[c[0] for c in CASES])
def test_forward_entry_points_write_only_their_outputs(moe, name, T, d, E, k, de, dtype):
    announce(f"canary forward {name} T={T} d={d} E={E} k={k} de={de} {dtype}")
    cfg = scaled_config("skewed" if dtype == "bf16" else "tiny_fp32", T=T, d_model=d, E=E, k=k, d_expert=de,
                        suffix="canary")
    inp = make_inputs(cfg, seed=21, device="cuda")
    x, wr, b, W1, W2 = inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"]
    tdt = x.dtype
    p = moe.make_problem(T, d, E, k, de, tdt)
    R = T * k
    ins = {"x": x, "w_router": wr, "W1": W1, "W2": W2}
    if b is not None:
        ins["bias"] = b
    before = {n: t.clone() for n, t in ins.items()}
    i32, f32 = torch.int32, torch.float32

    g = {"logits": Guarded((T, E), f32), "idx": Guarded((T, k), i32), "gate": Guarded((T, k), f32)}
    moe.moe_route(p, x, wr, b, g["logits"].t, g["idx"].t, g["gate"].t)
    check("moe_route", g, ins, before)

    g = {"logits": Guarded((T, E), f32), "idx": Guarded((T, k), i32), "gate": Guarded((T, k), f32),
         "ws": ws_guard(moe, p, moe.MOE_STAGE_ROUTE)}
    moe.moe_route_ws(p, x, wr, b, g["logits"].t, g["idx"].t, g["gate"].t, g["ws"].t)
    check("moe_route_ws", g, ins, before)
    idx, gate = g["idx"].t.clone(), g["gate"].t.clone()
    ins2 = dict(ins, idx=idx, gate=gate)
    before2 = dict(before, idx=idx.clone(), gate=gate.clone())

    g = {n: Guarded(s, i32) for n, s in (("counts", (E,)), ("offsets", (E + 1,)), ("perm", (R,)), ("inv", (R,)))}
    g["x_perm"] = Guarded((R, d), tdt)
    g["ws"] = ws_guard(moe, p, moe.MOE_STAGE_PERMUTE)
    moe.moe_permute(p, idx, x, g["counts"].t, g["offsets"].t, g["perm"].t, g["inv"].t, g["x_perm"].t, g["ws"].t)
    check("moe_permute", g, ins2, before2)
    offsets, perm, inv, x_perm = (g["offsets"].t.clone(), g["perm"].t.clone(), g["inv"].t.clone(),
                                  g["x_perm"].t.clone())

    g = {n: Guarded(s, i32) for n, s in (("counts", (E,)), ("offsets", (E + 1,)), ("perm", (R,)), ("inv", (R,)))}
    g["ws"] = ws_guard(moe, p, moe.MOE_STAGE_PERMUTE)
    moe.moe_permute_index(p, idx, g["counts"].t, g["offsets"].t, g["perm"].t, g["inv"].t, g["ws"].t)
    check("moe_permute_index", g, ins2, before2)

    g = {n: Guarded(s, i32) for n, s in (("counts", (E,)), ("offsets", (E + 1,)), ("perm", (R,)), ("inv", (R,)))}
    moe.moe_permute_index_noalloc(p, idx, g["counts"].t, g["offsets"].t, g["perm"].t, g["inv"].t)
    check("moe_permute_index_noalloc", g, ins2, before2)

    ins3 = dict(ins2, offsets=offsets, perm=perm, inv=inv, x_perm=x_perm)
    before3 = dict(before2, offsets=offsets.clone(), perm=perm.clone(), inv=inv.clone(), x_perm=x_perm.clone())
    g = {"y_perm": Guarded((R, d), tdt), "ws": ws_guard(moe, p, moe.MOE_STAGE_GROUPED_FFN)}
    moe.moe_grouped_ffn(p, x_perm, offsets, W1, W2, g["y_perm"].t, g["ws"].t)
    check("moe_grouped_ffn", g, ins3, before3)
    y_perm = g["y_perm"].t.clone()

    if dtype == "bf16":
        g = {"y_perm": Guarded((R, d), tdt), "ws": ws_guard(moe, p, moe.MOE_STAGE_GROUPED_FFN)}
        moe.moe_grouped_ffn_gather(p, x, perm, offsets, W1, W2, g["y_perm"].t, g["ws"].t)
        check("moe_grouped_ffn_gather", g, ins3, before3)
        assert torch.equal(g["y_perm"].t, y_perm)

    ins4 = dict(ins3, y_perm=y_perm)
    before4 = dict(before3, y_perm=y_perm.clone())
    g = {"y": Guarded((T, d), tdt)}
    moe.moe_combine(p, y_perm, inv, gate, g["y"].t)
    check("moe_combine", g, ins4, before4)
    y = g["y"].t.clone()

    for call in range(2):  # the second call finds the workspace as the first left it
        g = {"y": Guarded((T, d), tdt), "ws": ws_guard(moe, p, moe.MOE_STAGE_FORWARD)}
        moe.moe_forward(p, x, wr, b, W1, W2, g["y"].t, g["ws"].t)
        check("moe_forward", g, ins, before)
        assert torch.equal(g["y"].t, y), call


@pytest.mark.parametrize("T,d,E,k,de", [(300, 256, 16, 4, 320), (9, 512, 16, 2, 1024)], ids=["ragged", "decode"])
def test_training_entry_points_write_only_their_outputs(moe, T, d, E, k, de):
    announce(f"canary training T={T} d={d} E={E} k={k} de={de}")
    cfg = scaled_config("skewed", T=T, d_model=d, E=E, k=k, d_expert=de, suffix="canary")
    inp = make_inputs(cfg, seed=22, device="cuda")
    x, wr, b, W1, W2 = inp["x"], inp["w_router"], inp["router_bias"], inp["W1"], inp["W2"]
    dy = make_dense((T, d), 1.0, seed=22, tag=9, device="cuda")
    p = moe.make_problem(T, d, E, k, de, x.dtype)
    ins = {"x": x, "w_router": wr, "W1": W1, "W2": W2, "dy": dy}
    if b is not None:
        ins["bias"] = b
    before = {n: t.clone() for n, t in ins.items()}
    ws = ws_guard(moe, p, moe.MOE_STAGE_TRAIN)
    g = {"y": Guarded((T, d), x.dtype), "ws": ws}
    moe.moe_forward_train(p, x, wr, b, W1, W2, g["y"].t, ws.t)
    check("moe_forward_train", g, ins, before)
    bf, f32 = torch.bfloat16, torch.float32
    g = {"dx": Guarded((T, d), bf), "dw_router": Guarded((d, E), bf), "dbias": Guarded((E,), f32),
         "dW1": Guarded((E, d, de), bf), "dW2": Guarded((E, de, d), bf), "load_frac": Guarded((E,), f32),
         "mean_prob": Guarded((E,), f32), "ws": ws}
    moe.moe_backward(p, x, wr, W1, W2, dy, g["dx"].t, g["dw_router"].t, g["dbias"].t, g["dW1"].t, g["dW2"].t,
                     g["load_frac"].t, g["mean_prob"].t, ws.t)
    check("moe_backward", g, ins, before)


def test_guard_sees_a_write_next_to_the_tensor():
    """The bands catch a single byte written just before or just after the
    tensor (written here with torch, not by the library)."""
    for at in ("before", "after"):
        g = Guarded((3, 5), torch.bfloat16)
        assert g.intact()
        if at == "before":
            g.buf[BAND - 1] = 0
        else:
            g.buf[BAND + g.nbytes] = 0
        assert not g.intact(), at
