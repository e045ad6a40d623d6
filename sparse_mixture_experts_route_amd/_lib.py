"""ctypes declarations of libmoe.so and argument marshalling for its entry points."""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first: libmoe.so then binds to the HIP runtime torch already mapped

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_STAGE_PERMUTE = 0
MOE_STAGE_GROUPED_FFN = 1
MOE_STAGE_FORWARD = 2
MOE_STAGE_ROUTE = 3
MOE_STAGE_TRAIN = 4


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_str(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_expert", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class GemmPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tile", "bm", "bn", "bk", "grid", "k_steps", "max_split",
                                              "min_steps", "split_in_launch")] + \
               [("tiles", ctypes.c_int64)] + \
               [(n, ctypes.c_int32) for n in ("xcd_rounds", "xcd_leftover", "xcd_split", "split_xcds")]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("route_splits", "route_tokens_per_block", "route_fused_permute",
                                              "permute_form", "gather_in_gemm", "combine_streaming")] + \
               [("gemm", GemmPlan * 2), ("forward_one_launch", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_FILE):
        raise ImportError(f"{_LIB_FILE} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_FILE, mode=ctypes.RTLD_GLOBAL)
    P = ctypes.POINTER(Problem)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "moe_workspace_size": [P, i32, ctypes.POINTER(sz)],
        "moe_plan": [P, vp, ctypes.POINTER(Plan)],
        "moe_route": [P, vp, vp, vp, vp, vp, vp, vp],
        "moe_route_ws": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute": [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_grouped_ffn": [P, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute_index": [P, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute_index_noalloc": [P, vp, vp, vp, vp, vp, vp],
        "moe_grouped_ffn_gather": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_combine": [P, vp, vp, vp, vp, vp],
        "moe_forward": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_forward_train": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_backward": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    lib.moe_status_str.argtypes = [i32]
    lib.moe_status_str.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib_path() -> str:
    return _LIB_FILE


def moe_status_str(status: int) -> str:
    return _lib.moe_status_str(int(status)).decode()


def make_problem(T: int, d_model: int, E: int, k: int, d_expert: int, dtype) -> Problem:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}[dtype]
    elif isinstance(dtype, str):
        dtype = {"f32": MOE_DTYPE_F32, "bf16": MOE_DTYPE_BF16}[dtype]
    return Problem(int(T), int(d_model), int(E), int(k), int(d_expert), int(dtype))


def _ptr(t: Optional[torch.Tensor]):
    """Device address of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoe must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_workspace_size(p: Problem, stage: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.moe_workspace_size(ctypes.byref(p), int(stage), ctypes.byref(out)), "moe_workspace_size")
    return int(out.value)


def moe_plan(p: Problem, counts=None) -> dict:
    """The launch plan of problem p (host only). counts: E per-expert selection
    counts (any int sequence or CPU tensor) for the GEMMs' tile lists, or None."""
    buf = None
    if counts is not None:
        vals = [int(c) for c in (counts.tolist() if isinstance(counts, torch.Tensor) else counts)]
        if len(vals) != p.E:
            raise ValueError("counts must hold E entries")
        buf = (ctypes.c_int32 * p.E)(*vals)
    out = Plan()
    _check(_lib.moe_plan(ctypes.byref(p), ctypes.cast(buf, ctypes.c_void_p) if buf is not None else None,
                         ctypes.byref(out)), "moe_plan")
    d = {n: getattr(out, n) for n, _ in Plan._fields_ if n != "gemm"}
    d["gemm"] = [{n: getattr(g, n) for n, _ in GemmPlan._fields_} for g in out.gemm]
    return d


def moe_route(p: Problem, x, w_router, router_bias, logits, topk_idx, topk_gate, stream=None):
    _check(_lib.moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(logits),
                          _ptr(topk_idx), _ptr(topk_gate), _stream(stream)), "moe_route")


def moe_route_ws(p: Problem, x, w_router, router_bias, logits, topk_idx, topk_gate, ws, stream=None):
    _check(_lib.moe_route_ws(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(logits),
                             _ptr(topk_idx), _ptr(topk_gate), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "moe_route_ws")


def moe_permute(p: Problem, topk_idx, x, counts, offsets, perm, inv, x_perm, ws, stream=None):
    _check(_lib.moe_permute(ctypes.byref(p), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets), _ptr(perm),
                            _ptr(inv), _ptr(x_perm), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream)), "moe_permute")


def moe_grouped_ffn(p: Problem, x_perm, offsets, W1, W2, y_perm, ws, stream=None):
    _check(_lib.moe_grouped_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(W1), _ptr(W2), _ptr(y_perm),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_grouped_ffn")


def moe_permute_index(p: Problem, topk_idx, counts, offsets, perm, inv, ws, stream=None):
    _check(_lib.moe_permute_index(ctypes.byref(p), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                                  _ptr(inv), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_permute_index")


def moe_permute_index_noalloc(p: Problem, topk_idx, counts, offsets, perm, inv, stream=None):
    _check(_lib.moe_permute_index_noalloc(ctypes.byref(p), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                                          _ptr(inv), _stream(stream)), "moe_permute_index_noalloc")


def moe_grouped_ffn_gather(p: Problem, x, perm, offsets, W1, W2, y_perm, ws, stream=None):
    _check(_lib.moe_grouped_ffn_gather(ctypes.byref(p), _ptr(x), _ptr(perm), _ptr(offsets), _ptr(W1), _ptr(W2),
                                       _ptr(y_perm), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_grouped_ffn_gather")


def moe_combine(p: Problem, y_perm, inv, topk_gate, y, stream=None):
    _check(_lib.moe_combine(ctypes.byref(p), _ptr(y_perm), _ptr(inv), _ptr(topk_gate), _ptr(y),
                            _stream(stream)), "moe_combine")


def moe_forward(p: Problem, x, w_router, router_bias, W1, W2, y, ws, stream=None):
    _check(_lib.moe_forward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(W1), _ptr(W2),
                            _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


def moe_forward_train(p: Problem, x, w_router, router_bias, W1, W2, y, ws, stream=None):
    _check(_lib.moe_forward_train(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(W1), _ptr(W2),
                                  _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward_train")


def moe_backward(p: Problem, x, w_router, W1, W2, dy, dx, dw_router, dbias, dW1, dW2, load_frac, mean_prob, ws,
                 stream=None):
    _check(_lib.moe_backward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(W1), _ptr(W2), _ptr(dy), _ptr(dx),
                             _ptr(dw_router), _ptr(dbias), _ptr(dW1), _ptr(dW2), _ptr(load_frac), _ptr(mean_prob),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_backward")


def raw_lib():
    """The ctypes handle itself (for callers that pass raw addresses)."""
    return _lib
