"""Seeded synthetic inputs for the MoE layer (test and benchmark infrastructure).

This module only draws tensors: it holds none of the layer's arithmetic.  The
values come from ``gen.c`` (SplitMix64 counter streams, Box-Muller normals),
built on first use with gcc into ``libmoegen.so`` beside this file.

Workload shapes (the pages name the models, the shapes are public model
facts): DeepSeek-V3 has 256 routed experts with top-8 routing and one shared
expert (learn-kernels "Mixture-of-experts serving", first paragraph), model
width 7168 (llm-stack-book 7.13, "The Two Costs").  Every value is synthetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libmoegen.so")
_lib = None
_lock = threading.Lock()

# Tensor ids of the counter streams.
TID_X, TID_LOGITS, TID_BIAS, TID_W13, TID_W2, TID_WS13, TID_WS2, TID_PERM = 1, 2, 3, 4, 5, 6, 7, 8
TID_WR = 9


def build_lib(force: bool = False) -> str:
    """Compile gen.c into libmoegen.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build_lib()
            lib = ctypes.CDLL(_LIB_PATH)
            u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            lib.gen_bits.argtypes = [u64, u64, u64, i64, vp]
            lib.gen_normal_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
            lib.gen_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
            lib.gen_fp8_blocks.argtypes = [u64, u64, u64, i64, i64, dbl, dbl, vp, vp]
            lib.gen_permutation.argtypes = [u64, u64, ctypes.c_int32, vp]
            for f in (lib.gen_bits, lib.gen_normal_f32, lib.gen_normal_bf16, lib.gen_fp8_blocks,
                      lib.gen_permutation):
                f.restype = None
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def bits(seed: int, tid: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().gen_bits(seed, tid, offset, n, _ptr(out))
    return out


def normal_f32(seed: int, tid: int, shape, std: float, mean: float = 0.0, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().gen_normal_f32(seed, tid, offset, out.size, mean, std, _ptr(out))
    return out


def normal_bf16(seed: int, tid: int, shape, std: float, mean: float = 0.0, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of the same draws as normal_f32, rounded to nearest even."""
    out = np.empty(shape, dtype=np.uint16)
    _load().gen_normal_bf16(seed, tid, offset, out.size, mean, std, _ptr(out))
    return out


def fp8_blocks(seed: int, tid: int, rows: int, cols: int, std: float, offset: int = 0):
    """E4M3FN codes [rows][cols] (uint8) and per-128x128-block fp32 scales."""
    assert rows % 128 == 0 and cols % 128 == 0
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows // 128, cols // 128), dtype=np.float32)
    _load().gen_fp8_blocks(seed, tid, offset, rows, cols, 0.0, std, _ptr(codes), _ptr(scales))
    return codes, scales


def permutation(seed: int, tid: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().gen_permutation(seed, tid, n, _ptr(out))
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Storage decode of bf16 bit patterns (exact)."""
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    num_experts: int
    top_k: int
    d_model: int
    d_ff: int
    num_shared: int
    d_ff_shared: int
    n_group: int
    topk_group: int
    score: str          # "sigmoid" | "softmax"
    weight: str         # "norm_sum" | "softmax_selected"
    routed_scale: float
    act_dtype: str      # "f32" | "bf16"   (x and y)
    weight_dtype: str   # "f32" | "bf16" | "fp8"
    x_std: float
    w_std: float
    bias: str           # "none" | "zero" | "normal" | "zipf"
    bias_std: float = 0.0
    zipf_s: float = 1.1
    zipf_tau: float = 0.10
    tokens: tuple = field(default_factory=tuple)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # fp32 everywhere, 16 tokens, 8 experts top-2, softmax over the two
    # selected sigmoid scores, no shared expert, N(0, 0.02) data.
    "tiny": Workload("tiny", 8, 2, 256, 512, 0, 0, 1, 1, "sigmoid", "softmax_selected", 1.0,
                     "f32", "f32", 0.02, 0.02, "zero", tokens=(16,)),
    # Qwen3-30B-A3B-shaped decode layer: 128 experts, top-8 softmax routing.
    "qwen3": Workload("qwen3", 128, 8, 2048, 768, 0, 0, 1, 1, "softmax", "norm_sum", 1.0,
                      "bf16", "bf16", 1.0, 0.02, "none", tokens=(1, 8, 32, 128)),
    # DeepSeek-V3-shaped decode layer: sigmoid + bias, 8 groups / top-4 groups, x2.5.
    "dsv3": Workload("dsv3", 256, 8, 7168, 2048, 1, 2048, 8, 4, "sigmoid", "norm_sum", 2.5,
                     "bf16", "bf16", 1.0, 0.02, "normal", bias_std=0.1, tokens=(1, 8, 32, 128)),
    # Same layer, fp8 e4m3 expert weights with 128x128 block scales.
    "dsv3_fp8": Workload("dsv3_fp8", 256, 8, 7168, 2048, 1, 2048, 8, 4, "sigmoid", "norm_sum", 2.5,
                         "bf16", "fp8", 1.0, 0.02, "normal", bias_std=0.1, tokens=(32, 128, 512)),
    # Prefill: 4096 tokens, bias shaped for a Zipf(1.1) popularity skew.
    "dsv3_prefill": Workload("dsv3_prefill", 256, 8, 7168, 2048, 1, 2048, 8, 4, "sigmoid", "norm_sum",
                             2.5, "bf16", "bf16", 1.0, 0.02, "zipf", tokens=(4096,)),
}


def gen_x(w: Workload, T: int, seed: int = 0) -> np.ndarray:
    """Token activations [T][d]: fp32 values or bf16 bit patterns.  Row t uses
    stream indices t*d .. t*d+d-1, so a smaller T is a prefix of a larger one."""
    shape = (T, w.d_model)
    if w.act_dtype == "f32":
        return normal_f32(seed, TID_X, shape, w.x_std)
    return normal_bf16(seed, TID_X, shape, w.x_std)


def gen_logits(w: Workload, T: int, seed: int = 0) -> np.ndarray:
    """Router logits [T][E] fp32, N(0, 1)."""
    return normal_f32(seed, TID_LOGITS, (T, w.num_experts), 1.0)


def gen_router_weight(w: Workload, seed: int = 0) -> np.ndarray:
    """Router weight [E][d] in the activation dtype, N(0, 1/d): with N(0, 1)
    tokens the router logits come out about N(0, 1), the logit distribution
    of the decode workloads."""
    shape = (w.num_experts, w.d_model)
    std = float(1.0 / np.sqrt(w.d_model))
    if w.act_dtype == "f32":
        return normal_f32(seed, TID_WR, shape, std)
    return normal_bf16(seed, TID_WR, shape, std)


def gen_bias(w: Workload, seed: int = 0):
    """Per-expert routing bias [E] fp32, or None."""
    E = w.num_experts
    if w.bias == "none":
        return None
    if w.bias == "zero":
        return np.zeros(E, dtype=np.float32)
    if w.bias == "normal":
        return normal_f32(seed, TID_BIAS, (E,), w.bias_std)
    if w.bias == "zipf":
        # bias_e = tau * ln(r_e ** -s) with r a seeded random rank permutation
        # (1 = most popular): popularity falls off with rank like a power law.
        rank = permutation(seed, TID_PERM, E).astype(np.float64) + 1.0
        return (w.zipf_tau * (-w.zipf_s) * np.log(rank)).astype(np.float32)
    raise ValueError(w.bias)


def _w_rows_cols(w: Workload, which: str):
    d, F, Fs = w.d_model, w.d_ff, w.d_ff_shared
    return {"w13": (2 * F, d), "w2": (d, F), "ws13": (2 * Fs, d), "ws2": (d, Fs)}[which]


_TIDS = {"w13": TID_W13, "w2": TID_W2, "ws13": TID_WS13, "ws2": TID_WS2}


def gen_weight(w: Workload, which: str, expert: int = 0, seed: int = 0):
    """One expert's matrix.  which: 'w13' [2F][d] (rows [0,F) gate, [F,2F) up),
    'w2' [d][F], 'ws13' [2Fs][d], 'ws2' [d][Fs] (shared expert, expert=0).

    Returns fp32 array, bf16 bit patterns, or (fp8 codes, block scales)."""
    rows, cols = _w_rows_cols(w, which)
    off = expert * rows * cols
    tid = _TIDS[which]
    if w.weight_dtype == "f32":
        return normal_f32(seed, tid, (rows, cols), w.w_std, offset=off)
    if w.weight_dtype == "bf16":
        return normal_bf16(seed, tid, (rows, cols), w.w_std, offset=off)
    return fp8_blocks(seed, tid, rows, cols, w.w_std, offset=off)
