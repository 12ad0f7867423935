"""ctypes binding of libmoe.so: argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors (or raw device addresses as ints, or None for NULL) and passes their
addresses and the current HIP stream through.  No step of the layer runs in
Python: if libmoe.so is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MOE_FMT_NVFP4 = 1
MOE_FMT_MXFP4 = 2
MOE_FMT_FP8_B128 = 3
MOE_FMT_MXFP8 = 4

MOE_OP_GATE_UP_SWIGLU = 0
MOE_OP_DOWN = 1

MOE_ACT_EXACT = 0
MOE_ACT_MXFP8 = 1
MOE_ACT_MXFP4 = 2
MOE_ACT_FP8_T128 = 3

EXPORTED = ["moe_abi_version", "moe_status_string", "moe_last_error", "moe_validate_layer", "moe_workspace_size",
            "moe_route_topk", "moe_permute_workspace_size", "moe_permute", "moe_expert_gemm",
            "moe_combine", "moe_layer_forward", "moe_quantize_act", "moe_expert_gemm_q",
            "moe_layer_forward_ex", "moe_route_table", "moe_layer_forward_routed",
            "moe_noalloc_workspace_limit", "moe_layer_forward_noalloc", "moe_decode_gate_up"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = ""
        if status == MOE_ERR_HIP:
            detail = ": " + LIB.moe_last_error().decode()
        super().__init__(f"{where} failed: {status} ({status_string(status)}{detail})")


class moe_qweight(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p),
                ("expert_stride_codes", ctypes.c_int64), ("expert_stride_scales", ctypes.c_int64)]


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", moe_qweight), ("up", moe_qweight), ("down", moe_qweight),
                ("has_shared", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("sh_gate", moe_qweight), ("sh_up", moe_qweight), ("sh_down", moe_qweight)]


def _load():
    # torch owns device memory and streams; load its HIP runtime first so that
    # libmoe.so binds to that same runtime (one runtime per process).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m quantized_moe_expert_02_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP = ctypes.POINTER(moe_layer_desc)
    sig = {
        "moe_abi_version": (I32, []),
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_validate_layer": (I32, [LP]),
        "moe_workspace_size": (SZ, [LP, I32]),
        "moe_route_topk": (I32, [LP, P, P, I32, P, P, P, SZ, P]),
        "moe_permute_workspace_size": (SZ, [I32, I32, I32]),
        "moe_permute": (I32, [P, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
        "moe_expert_gemm": (I32, [I32, LP, I32, P, P, P, I32, P, P, P, SZ, P]),
        "moe_combine": (I32, [P, P, P, P, I32, I32, I32, P, P]),
        "moe_layer_forward": (I32, [LP, P, I32, P, P, SZ, P, P, P, P]),
        "moe_quantize_act": (I32, [I32, P, I32, I32, P, P, P]),
        "moe_expert_gemm_q": (I32, [I32, I32, LP, I32, P, P, P, I32, P, P, P, P, SZ, P]),
        "moe_layer_forward_ex": (I32, [LP, P, I32, P, P, SZ, I32, P, P, P, P]),
        "moe_route_table": (I32, [LP, P, P, P, P, I32, I32, P, P, P, SZ, P]),
        "moe_layer_forward_routed": (I32, [LP, P, I32, P, P, P, P, SZ, I32, P]),
        "moe_noalloc_workspace_limit": (SZ, []),
        "moe_layer_forward_noalloc": (I32, [LP, P, I32, P, P]),
        "moe_decode_gate_up": (I32, [LP, P, I32, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def _p(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(status: int, where: str) -> int:
    if status != MOE_OK:
        raise MoeError(status, where)
    return status


def status_string(status: int) -> str:
    return LIB.moe_status_string(status).decode()


def moe_abi_version() -> int:
    return LIB.moe_abi_version()


def moe_validate_layer(L: moe_layer_desc) -> int:
    return LIB.moe_validate_layer(ctypes.byref(L))


def moe_workspace_size(L: moe_layer_desc, T: int) -> int:
    return LIB.moe_workspace_size(ctypes.byref(L), T)


def moe_permute_workspace_size(T: int, k: int, E: int) -> int:
    return LIB.moe_permute_workspace_size(T, k, E)


def moe_route_topk(L, x, logits, T, topk_ids, topk_w, ws, ws_bytes=None, stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_route_topk(ctypes.byref(L), _p(x), _p(logits), T, _p(topk_ids), _p(topk_w), _p(ws),
                            wsb, _stream(stream))
    return _check(st, "moe_route_topk") if check else st


def moe_permute(topk_ids, T, k, E, counts, offsets, perm_to_pair, pair_to_perm, active_experts, ws,
                ws_bytes=None, stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_permute(_p(topk_ids), T, k, E, _p(counts), _p(offsets), _p(perm_to_pair),
                         _p(pair_to_perm), _p(active_experts), _p(ws), wsb, _stream(stream))
    return _check(st, "moe_permute") if check else st


def moe_expert_gemm(op, L, shared, offsets, perm_to_pair, active_experts, T, inp, out, ws,
                    ws_bytes=None, stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_expert_gemm(op, ctypes.byref(L), shared, _p(offsets), _p(perm_to_pair),
                             _p(active_experts), T, _p(inp), _p(out), _p(ws), wsb, _stream(stream))
    return _check(st, "moe_expert_gemm") if check else st


def moe_combine(y_perm, topk_w, pair_to_perm, y_shared, T, k, H, out, stream=None, check=True):
    st = LIB.moe_combine(_p(y_perm), _p(topk_w), _p(pair_to_perm), _p(y_shared), T, k, H, _p(out),
                         _stream(stream))
    return _check(st, "moe_combine") if check else st


def moe_layer_forward(L, x, T, out, ws, ws_bytes=None, dbg_logits=None, dbg_ids=None, dbg_w=None,
                      stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_layer_forward(ctypes.byref(L), _p(x), T, _p(out), _p(ws), wsb, _p(dbg_logits),
                               _p(dbg_ids), _p(dbg_w), _stream(stream))
    return _check(st, "moe_layer_forward") if check else st


def moe_layer_forward_ex(L, x, T, out, ws, act_mode, ws_bytes=None, dbg_logits=None, dbg_ids=None,
                         dbg_w=None, stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_layer_forward_ex(ctypes.byref(L), _p(x), T, _p(out), _p(ws), wsb, act_mode,
                                  _p(dbg_logits), _p(dbg_ids), _p(dbg_w), _stream(stream))
    return _check(st, "moe_layer_forward_ex") if check else st


def moe_quantize_act(mode, inp, rows, K, codes, scales, stream=None, check=True):
    st = LIB.moe_quantize_act(mode, _p(inp), rows, K, _p(codes), _p(scales), _stream(stream))
    return _check(st, "moe_quantize_act") if check else st


def moe_expert_gemm_q(mode, op, L, shared, offsets, perm_to_pair, active_experts, T, in_codes,
                      in_scales, out, ws, ws_bytes=None, stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_expert_gemm_q(mode, op, ctypes.byref(L), shared, _p(offsets), _p(perm_to_pair),
                               _p(active_experts), T, _p(in_codes), _p(in_scales), _p(out), _p(ws),
                               wsb, _stream(stream))
    return _check(st, "moe_expert_gemm_q") if check else st


def moe_route_table(L, x, logits, token_ids, table, V, T, topk_ids, topk_w, ws, ws_bytes=None,
                    stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_route_table(ctypes.byref(L), _p(x), _p(logits), _p(token_ids), _p(table), V, T,
                             _p(topk_ids), _p(topk_w), _p(ws), wsb, _stream(stream))
    return _check(st, "moe_route_table") if check else st


def moe_layer_forward_routed(L, x, T, topk_ids, topk_w, out, ws, act_mode=0, ws_bytes=None,
                             stream=None, check=True):
    wsb = ws_bytes if ws_bytes is not None else (ws.numel() * ws.element_size() if ws is not None else 0)
    st = LIB.moe_layer_forward_routed(ctypes.byref(L), _p(x), T, _p(topk_ids), _p(topk_w), _p(out),
                                      _p(ws), wsb, act_mode, _stream(stream))
    return _check(st, "moe_layer_forward_routed") if check else st


def moe_noalloc_workspace_limit() -> int:
    return LIB.moe_noalloc_workspace_limit()


def moe_layer_forward_noalloc(L, x, T, out, stream=None, check=True):
    st = LIB.moe_layer_forward_noalloc(ctypes.byref(L), _p(x), T, _p(out), _stream(stream))
    return _check(st, "moe_layer_forward_noalloc") if check else st


def moe_decode_gate_up(L, x, T, topk_ids, h, h_shared, stream=None, check=True):
    st = LIB.moe_decode_gate_up(ctypes.byref(L), _p(x), T, _p(topk_ids), _p(h), _p(h_shared),
                                _stream(stream))
    return _check(st, "moe_decode_gate_up") if check else st
