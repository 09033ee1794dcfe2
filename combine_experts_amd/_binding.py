"""ctypes binding of libmoe_hip.so: argument marshalling only.

Every function has the name and argument order of the C entry point it
wraps (see include/moe.h).  Pointer arguments accept a torch tensor (its
data_ptr()), a plain integer address, or None (NULL).  `stream` accepts a
torch.cuda.Stream, a raw hipStream_t integer, or None for torch's current
stream.  A non-OK status raises MoeError.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP, MOE_ERR_SCRATCH_LIMIT = range(6)
SCORE = {"softmax": 0, "sigmoid": 1}
WEIGHT = {"norm_sum": 0, "softmax_selected": 1}
DTYPE = {"f32": 0, "bf16": 1, "fp8": 2}

_c_i32, _c_vp = ctypes.c_int32, ctypes.c_void_p


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("num_experts", _c_i32), ("top_k", _c_i32), ("d_model", _c_i32), ("d_ff", _c_i32),
        ("num_shared", _c_i32), ("d_ff_shared", _c_i32), ("n_group", _c_i32), ("topk_group", _c_i32),
        ("score_fn", _c_i32), ("weight_fn", _c_i32), ("routed_scale", ctypes.c_float),
        ("act_dtype", _c_i32), ("weight_dtype", _c_i32), ("masked_layout", _c_i32),
    ]


class MoeWeights(ctypes.Structure):
    _fields_ = [
        ("w13", _c_vp), ("w2", _c_vp), ("ws13", _c_vp), ("ws2", _c_vp),
        ("w13_scale", _c_vp), ("w2_scale", _c_vp), ("ws13_scale", _c_vp), ("ws2_scale", _c_vp),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library():
    """Load libmoe_hip.so (built in-tree); raise ImportError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python combine_experts_amd/build.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    cp = ctypes.POINTER(MoeConfig)
    wp = ctypes.POINTER(MoeWeights)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.moe_dispatch_rows.argtypes = [cp, i32]
    lib.moe_dispatch_rows.restype = ctypes.c_int64
    lib.moe_ffn_workspace_size.argtypes = [cp, i32]
    lib.moe_ffn_workspace_size.restype = sz
    lib.moe_workspace_size.argtypes = [cp, i32]
    lib.moe_workspace_size.restype = sz
    lib.moe_route.argtypes = [cp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_dispatch.argtypes = [cp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_route_dispatch.argtypes = [cp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_expert_ffn.argtypes = [cp, i32, vp, vp, vp, wp, vp, vp, vp, vp, sz, vp]
    lib.moe_ffn_gate_up.argtypes = [cp, i32, vp, vp, vp, wp, vp, vp, sz, vp]
    lib.moe_ffn_down.argtypes = [cp, i32, vp, wp, vp, sz, vp, vp, vp]
    lib.moe_combine.argtypes = [cp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_layer.argtypes = [cp, i32, vp, vp, vp, wp, vp, vp, sz, vp]
    lib.moe_router_logits.argtypes = [cp, i32, vp, vp, vp, vp]
    lib.moe_router_logits_ws.argtypes = [cp, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_router_workspace_size.argtypes = [cp, i32]
    lib.moe_router_workspace_size.restype = sz
    lib.moe_layer_fused.argtypes = [cp, i32, vp, vp, vp, vp, wp, vp, vp, sz, vp]
    lib.moe_fused_workspace_size.argtypes = [cp, i32]
    lib.moe_fused_workspace_size.restype = sz
    lib.moe_fused_supported.argtypes = [cp, i32]
    lib.moe_fused_supported.restype = i32
    lib.moe_layer_static.argtypes = [cp, i32, vp, vp, vp, wp, vp, vp]
    lib.moe_layer_static_max_bytes.argtypes = []
    lib.moe_layer_static_max_bytes.restype = sz
    for f in (lib.moe_layer_fused, lib.moe_layer_static, lib.moe_route, lib.moe_dispatch, lib.moe_route_dispatch, lib.moe_expert_ffn, lib.moe_ffn_gate_up,
              lib.moe_ffn_down, lib.moe_combine, lib.moe_layer, lib.moe_router_logits, lib.moe_router_logits_ws):
        f.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_config(num_experts, top_k, d_model, d_ff, num_shared=0, d_ff_shared=0, n_group=1, topk_group=1,
                score="sigmoid", weight="norm_sum", routed_scale=1.0, act_dtype="bf16",
                weight_dtype="bf16", masked=False) -> MoeConfig:
    """Build a moe_config from names ('sigmoid'/'softmax', 'norm_sum'/'softmax_selected',
    'f32'/'bf16'/'fp8'); masked selects the masked dispatch layout."""
    return MoeConfig(num_experts, top_k, d_model, d_ff, num_shared, d_ff_shared, n_group, topk_group,
                     SCORE[score], WEIGHT[weight], float(routed_scale), DTYPE[act_dtype],
                     DTYPE[weight_dtype], 1 if masked else 0)


def make_weights(w13, w2, ws13=None, ws2=None, w13_scale=None, w2_scale=None, ws13_scale=None,
                 ws2_scale=None) -> MoeWeights:
    return MoeWeights(*[_ptr(a) for a in (w13, w2, ws13, ws2, w13_scale, w2_scale, ws13_scale, ws2_scale)])


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load_library().moe_status_string(status).decode())


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_dispatch_rows(cfg: MoeConfig, T: int) -> int:
    return load_library().moe_dispatch_rows(ctypes.byref(cfg), T)


def moe_ffn_workspace_size(cfg: MoeConfig, max_tokens: int) -> int:
    return load_library().moe_ffn_workspace_size(ctypes.byref(cfg), max_tokens)


def moe_workspace_size(cfg: MoeConfig, max_tokens: int) -> int:
    return load_library().moe_workspace_size(ctypes.byref(cfg), max_tokens)


def moe_route(cfg, T, logits, bias, topk_idx, topk_w, expert_count, ticket, stream=None):
    _check(load_library().moe_route(ctypes.byref(cfg), T, _ptr(logits), _ptr(bias), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(expert_count), _ptr(ticket), _stream(stream)))


def moe_dispatch(cfg, T, x, topk_idx, expert_count, ticket, recv, recv_scale, expert_offset, row_of,
                 stream=None):
    _check(load_library().moe_dispatch(ctypes.byref(cfg), T, _ptr(x), _ptr(topk_idx), _ptr(expert_count),
                                       _ptr(ticket), _ptr(recv), _ptr(recv_scale), _ptr(expert_offset),
                                       _ptr(row_of), _stream(stream)))


def moe_route_dispatch(cfg, T, logits, bias, x, topk_idx, topk_w, expert_count, ticket, recv, recv_scale,
                       row_of, stream=None):
    _check(load_library().moe_route_dispatch(ctypes.byref(cfg), T, _ptr(logits), _ptr(bias), _ptr(x),
                                             _ptr(topk_idx), _ptr(topk_w), _ptr(expert_count), _ptr(ticket),
                                             _ptr(recv), _ptr(recv_scale), _ptr(row_of), _stream(stream)))


def moe_expert_ffn(cfg, T, recv, recv_scale, expert_offset, weights: MoeWeights, x, expert_out, shared_out,
                   ws, ws_bytes, stream=None):
    _check(load_library().moe_expert_ffn(ctypes.byref(cfg), T, _ptr(recv), _ptr(recv_scale),
                                         _ptr(expert_offset), ctypes.byref(weights), _ptr(x), _ptr(expert_out),
                                         _ptr(shared_out), _ptr(ws), ws_bytes, _stream(stream)))


def moe_ffn_gate_up(cfg, T, recv, recv_scale, expert_offset, weights: MoeWeights, x, ws, ws_bytes, stream=None):
    _check(load_library().moe_ffn_gate_up(ctypes.byref(cfg), T, _ptr(recv), _ptr(recv_scale),
                                          _ptr(expert_offset), ctypes.byref(weights), _ptr(x), _ptr(ws),
                                          ws_bytes, _stream(stream)))


def moe_ffn_down(cfg, T, expert_offset, weights: MoeWeights, ws, ws_bytes, expert_out, shared_out, stream=None):
    _check(load_library().moe_ffn_down(ctypes.byref(cfg), T, _ptr(expert_offset), ctypes.byref(weights),
                                       _ptr(ws), ws_bytes, _ptr(expert_out), _ptr(shared_out), _stream(stream)))


def moe_combine(cfg, T, expert_out, row_of, topk_w, shared_out, y, expert_count, stream=None):
    _check(load_library().moe_combine(ctypes.byref(cfg), T, _ptr(expert_out), _ptr(row_of), _ptr(topk_w),
                                      _ptr(shared_out), _ptr(y), _ptr(expert_count), _stream(stream)))


def moe_layer(cfg, T, x, logits, bias, weights: MoeWeights, y, ws, ws_bytes, stream=None):
    _check(load_library().moe_layer(ctypes.byref(cfg), T, _ptr(x), _ptr(logits), _ptr(bias),
                                    ctypes.byref(weights), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)))


def moe_router_logits(cfg, T, x, w_router, logits, stream=None):
    _check(load_library().moe_router_logits(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(logits),
                                            _stream(stream)))


def moe_router_logits_ws(cfg, T, x, w_router, logits, ws, ws_bytes, stream=None):
    _check(load_library().moe_router_logits_ws(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(logits),
                                               _ptr(ws), ws_bytes, _stream(stream)))


def moe_router_workspace_size(cfg: MoeConfig, max_tokens: int) -> int:
    return load_library().moe_router_workspace_size(ctypes.byref(cfg), max_tokens)


def moe_layer_static(cfg, T, x, logits, bias, weights: MoeWeights, y, stream=None):
    _check(load_library().moe_layer_static(ctypes.byref(cfg), T, _ptr(x), _ptr(logits), _ptr(bias),
                                           ctypes.byref(weights), _ptr(y), _stream(stream)))


def moe_layer_static_max_bytes() -> int:
    return load_library().moe_layer_static_max_bytes()


def moe_layer_fused(cfg, T, x, logits, w_router, bias, weights: MoeWeights, y, ws, ws_bytes, stream=None):
    _check(load_library().moe_layer_fused(ctypes.byref(cfg), T, _ptr(x), _ptr(logits), _ptr(w_router), _ptr(bias),
                                          ctypes.byref(weights), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)))


def moe_fused_workspace_size(cfg: MoeConfig, max_tokens: int) -> int:
    return load_library().moe_fused_workspace_size(ctypes.byref(cfg), max_tokens)


def moe_fused_supported(cfg: MoeConfig, T: int) -> bool:
    return bool(load_library().moe_fused_supported(ctypes.byref(cfg), T))
