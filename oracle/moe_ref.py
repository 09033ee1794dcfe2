"""ctypes binding of the C++ CPU oracle (libmoe_ref.so, built from moe_ref.cpp).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` load it.  It shares no code with the GPU
library and imports nothing from it or from the numpy oracle.

Besides the raw entry points (``lib()``), this module exposes the same
functions as the numpy oracle (``route``, ``dispatch``, ``combine``,
``swiglu_expert``, ``layer``, ``dense_token``, ``router_logits``, the E4M3
codec), taking float64 weights through ``get_expert`` callbacks, so that the
oracle pins run against both implementations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_ref.cpp")
_HDR = os.path.join(_HERE, "moe_ref.h")
LIB_PATH = os.path.join(_HERE, "libmoe_ref.so")
_lib = None
_lock = threading.Lock()

F32, BF16, E4M3, F64 = 0, 1, 2, 3
_DT = {"f32": F32, "bf16": BF16, "fp8": E4M3, "f64": F64}


class RefConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_experts", "top_k", "d_model", "d_ff", "num_shared",
                                              "d_ff_shared", "n_group", "topk_group", "score_fn", "weight_fn")]
    _fields_ += [("routed_scale", ctypes.c_double), ("act_dtype", ctypes.c_int32),
                 ("weight_dtype", ctypes.c_int32), ("act_quant", ctypes.c_int32)]


class RefWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w13", "w2", "ws13", "ws2", "w13_scale", "w2_scale",
                                               "ws13_scale", "ws2_scale")]


def build_lib(force: bool = False) -> str:
    """Compile moe_ref.cpp with g++ (no fused multiply-adds, no fast math)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < newest:
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                               "-fno-fast-math", _SRC, "-o", tmp])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build_lib()
            L = ctypes.CDLL(LIB_PATH)
            cp, wp = ctypes.POINTER(RefConfig), ctypes.POINTER(RefWeights)
            i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
            sig = {
                "moe_ref_keys": [cp, i32, vp, vp, vp],
                "moe_ref_route": [cp, i32, vp, vp, vp, vp],
                "moe_ref_gate_weights": [cp, i32, vp, vp, vp],
                "moe_ref_margins": [cp, i32, vp, vp, vp],
                "moe_ref_dispatch": [cp, i32, vp, vp, vp, vp, vp],
                "moe_ref_gather": [cp, i32, vp, vp, vp],
                "moe_ref_expert_ffn": [cp, i32, vp, vp, wp, vp, vp, vp, i32],
                "moe_ref_combine": [cp, i32, vp, vp, vp, vp, vp],
                "moe_ref_layer": [cp, i32, vp, vp, vp, wp, vp, vp, vp, i32],
                "moe_ref_dense_token": [cp, vp, vp, vp, wp, vp],
                "moe_ref_router_logits": [cp, i32, vp, vp, vp],
                "moe_ref_quantize_rows": [i64, i64, vp, vp, vp],
            }
            for name, args in sig.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = ctypes.c_int
            L.moe_ref_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.moe_ref_e4m3_decode.restype = ctypes.c_double
            L.moe_ref_e4m3_encode.argtypes = [ctypes.c_float]
            L.moe_ref_e4m3_encode.restype = ctypes.c_uint8
            _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be contiguous"
    return a.ctypes.data


def _ok(status):
    if status != 0:
        raise ValueError("moe_ref: invalid argument")


def config(spec, d_model=1, d_ff=1, d_ff_shared=0, act_dtype="f64", weight_dtype="f64", act_quant=False):
    """moe_ref_config of a workload-like spec (num_experts, top_k, n_group,
    topk_group, score, weight, routed_scale, num_shared)."""
    ns = int(getattr(spec, "num_shared", 0) or 0) if d_ff_shared > 0 else 0
    return RefConfig(spec.num_experts, spec.top_k, d_model, d_ff, ns, d_ff_shared if ns else 0,
                     spec.n_group, spec.topk_group, 1 if spec.score == "sigmoid" else 0,
                     0 if spec.weight == "norm_sum" else 1, float(spec.routed_scale), _DT[act_dtype],
                     _DT[weight_dtype], 1 if act_quant else 0)


# ---------------------------------------------------------------------------
# The numpy oracle's interface, on the C++ implementation
# ---------------------------------------------------------------------------


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def route(logits, bias, spec):
    logits = _f32(logits)
    T, E = logits.shape
    c = config(spec)
    idx = np.empty((T, spec.top_k), np.int32)
    w = np.empty((T, spec.top_k), np.float64)
    b = _f32(bias) if bias is not None else None
    _ok(lib().moe_ref_route(ctypes.byref(c), T, _p(logits), _p(b), _p(idx), _p(w)))
    keys = np.empty((T, E), np.float32)
    _ok(lib().moe_ref_keys(ctypes.byref(c), T, _p(logits), _p(b), _p(keys)))
    return idx, w, {"keys": keys, "logits": logits, "bias": b}


def gate_weights(logits, idx, spec):
    logits = _f32(logits)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    c = config(spec)
    w = np.empty(idx.shape, np.float64)
    _ok(lib().moe_ref_gate_weights(ctypes.byref(c), idx.shape[0], _p(logits), _p(idx), _p(w)))
    return w


def routing_margins(info, spec):
    logits = info["logits"]
    c = config(spec)
    gap = np.empty(logits.shape[0], np.float64)
    _ok(lib().moe_ref_margins(ctypes.byref(c), logits.shape[0], _p(logits), _p(info["bias"]), _p(gap)))
    return gap


class _Spec:
    def __init__(self, E, k):
        self.num_experts, self.top_k, self.n_group, self.topk_group = E, k, 1, 1
        self.score, self.weight, self.routed_scale, self.num_shared = "sigmoid", "norm_sum", 1.0, 0


def dispatch(idx, num_experts):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    c = config(_Spec(num_experts, k))
    counts = np.empty(num_experts, np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    row_of = np.empty((T, k), np.int32)
    tok = np.empty(T * k, np.int32)
    _ok(lib().moe_ref_dispatch(ctypes.byref(c), T, _p(idx), _p(counts), _p(offsets), _p(row_of), _p(tok)))
    return counts.astype(np.int64), offsets.astype(np.int64), row_of.astype(np.int64), tok.astype(np.int64)


def gather_rows(x, token_of_row):
    x = _f64(x)
    tok = np.ascontiguousarray(token_of_row, dtype=np.int32)
    T, d = x.shape
    spec = _Spec(1, 1)
    c = config(spec, d_model=d)
    c.top_k = 1
    recv = np.empty((len(tok), d), np.float64)
    # one "token slot" per row: gather with a k = 1 view of the rows
    _ok(lib().moe_ref_gather(ctypes.byref(c), len(tok), _p(x), _p(tok), _p(recv)))
    return recv


def combine(expert_out, row_of, w, shared_out=None):
    eout = _f64(expert_out)
    row_of = np.ascontiguousarray(row_of, dtype=np.int32)
    T, k = row_of.shape
    d = eout.shape[1]
    spec = _Spec(max(k, 1), k)
    c = config(spec, d_model=d)
    y = np.empty((T, d), np.float64)
    _ok(lib().moe_ref_combine(ctypes.byref(c), T, _p(eout), _p(row_of), _p(_f64(w)),
                              _p(_f64(shared_out)) if shared_out is not None else None, _p(y)))
    return y


def _weights_f64(get_expert, E, get_shared=None):
    w13 = _f64(np.stack([get_expert(e)[0] for e in range(E)]))
    w2 = _f64(np.stack([get_expert(e)[1] for e in range(E)]))
    keep = [w13, w2]
    W = RefWeights(_p(w13), _p(w2), None, None, None, None, None, None)
    if get_shared is not None:
        ws13, ws2 = (_f64(a) for a in get_shared())
        keep += [ws13, ws2]
        W.ws13, W.ws2 = _p(ws13), _p(ws2)
    return W, keep


def swiglu_expert(a, w13, w2, act_quant=False):
    a = _f64(a)
    n, d = a.shape
    w13, w2 = _f64(w13), _f64(w2)
    F = w13.shape[0] // 2
    spec = _Spec(1, 1)
    c = config(spec, d_model=d, d_ff=F, act_quant=act_quant)
    W = RefWeights(_p(w13), _p(w2), None, None, None, None, None, None)
    out = np.empty((n, d), np.float64)
    offsets = np.array([0, n], np.int32)
    _ok(lib().moe_ref_expert_ffn(ctypes.byref(c), n, _p(a), _p(offsets), ctypes.byref(W), None, _p(out), None, 1))
    return out


def layer(x, logits, bias, spec, get_expert, get_shared=None, idx=None, w=None, act_quant=False, nthreads=1):
    x = _f64(x)
    T, d = x.shape
    E = spec.num_experts
    w13_0 = np.asarray(get_expert(0)[0])
    F = w13_0.shape[0] // 2
    shared = bool(getattr(spec, "num_shared", 0)) and get_shared is not None
    Fs = np.asarray(get_shared()[0]).shape[0] // 2 if shared else 0
    c = config(spec, d_model=d, d_ff=F, d_ff_shared=Fs, act_quant=act_quant)
    c.num_shared = 1 if shared else 0
    W, keep = _weights_f64(get_expert, E, get_shared if shared else None)
    y = np.empty((T, d), np.float64)
    lg = _f32(logits) if logits is not None else None
    b = _f32(bias) if bias is not None else None
    ii = np.ascontiguousarray(idx, dtype=np.int32) if idx is not None else None
    ww = _f64(w) if w is not None else None
    _ok(lib().moe_ref_layer(ctypes.byref(c), T, _p(x), _p(lg), _p(b), ctypes.byref(W), _p(ii), _p(ww), _p(y),
                            nthreads))
    del keep
    return y


def dense_token(x_t, idx_t, w_t, get_expert, get_shared=None, act_quant=False):
    x_t = _f64(x_t)
    d = x_t.shape[0]
    idx_t = np.ascontiguousarray(idx_t, dtype=np.int32)
    k = len(idx_t)
    E = int(idx_t.max()) + 1
    F = np.asarray(get_expert(int(idx_t[0]))[0]).shape[0] // 2
    Fs = np.asarray(get_shared()[0]).shape[0] // 2 if get_shared is not None else 0
    spec = _Spec(max(E, k), k)
    spec.num_shared = 1 if get_shared is not None else 0
    c = config(spec, d_model=d, d_ff=F, d_ff_shared=Fs, act_quant=act_quant)
    # only the token's experts are read; the others are zero-filled placeholders
    zero = (np.zeros((2 * F, d)), np.zeros((d, F)))
    picked = set(int(e) for e in idx_t)
    W, keep = _weights_f64(lambda e: get_expert(e) if e in picked else zero, spec.num_experts, get_shared)
    y = np.empty(d, np.float64)
    _ok(lib().moe_ref_dense_token(ctypes.byref(c), _p(x_t), _p(idx_t), _p(_f64(w_t)), ctypes.byref(W), _p(y)))
    del keep
    return y


def router_logits(x, w_router):
    x, wr = _f64(x), _f64(w_router)
    T, d = x.shape
    E = wr.shape[0]
    spec = _Spec(E, 1)
    c = config(spec, d_model=d)
    out = np.empty((T, E), np.float64)
    _ok(lib().moe_ref_router_logits(ctypes.byref(c), T, _p(x), _p(wr), _p(out)))
    return out


def e4m3_decode(codes):
    c = np.asarray(codes, dtype=np.uint8)
    f = lib().moe_ref_e4m3_decode
    return np.array([f(int(v)) for v in c.reshape(-1)], np.float64).reshape(c.shape)


def e4m3_encode(v32):
    v = np.asarray(v32, dtype=np.float32)
    f = lib().moe_ref_e4m3_encode
    return np.array([f(float(a)) for a in v.reshape(-1)], np.uint8).reshape(v.shape)


def quantize_rows_1x128(x32):
    x32 = _f32(x32)
    n, d = x32.shape
    codes = np.empty((n, d), np.uint8)
    scales = np.empty((n, d // 128), np.float32)
    _ok(lib().moe_ref_quantize_rows(n, d, _p(x32), _p(codes), _p(scales)))
    return codes, scales


def dequant_rows_1x128(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    return e4m3_decode(codes) * np.repeat(np.asarray(scales, dtype=np.float64), 128, axis=1)


def selection_keys(logits, bias, score):
    logits = _f32(logits)
    T, E = logits.shape
    spec = _Spec(E, 1)
    spec.score = score
    c = config(spec)
    keys = np.empty((T, E), np.float32)
    b = _f32(bias) if bias is not None else None
    _ok(lib().moe_ref_keys(ctypes.byref(c), T, _p(logits), _p(b), _p(keys)))
    return keys


def swiglu_storage(a, w13, w2, weight_dtype, w13_scale=None, w2_scale=None, act_quant=False, nthreads=0):
    """One expert on float64 rows a [n][d], its weights in storage form
    (float32 values, bf16 bits as uint16, or E4M3 codes with 128x128 block
    scales): out[r] = W2 (silu(Wg a_r) * (Wu a_r)), accumulated in double."""
    a = _f64(a)
    n, d = a.shape
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    F = w13.shape[0] // 2
    c = config(_Spec(1, 1), d_model=d, d_ff=F, weight_dtype=weight_dtype, act_quant=act_quant)
    s13 = np.ascontiguousarray(w13_scale, dtype=np.float32) if w13_scale is not None else None
    s2 = np.ascontiguousarray(w2_scale, dtype=np.float32) if w2_scale is not None else None
    W = RefWeights(_p(w13), _p(w2), None, None, _p(s13), _p(s2), None, None)
    out = np.empty((n, d), np.float64)
    offsets = np.array([0, n], np.int32)
    _ok(lib().moe_ref_expert_ffn(ctypes.byref(c), n, _p(a), _p(offsets), ctypes.byref(W), None, _p(out), None,
                                 nthreads))
    return out
