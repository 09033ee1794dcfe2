#!/usr/bin/env python3
"""Benchmark of the MoE layer on one MI355X.

One step = one moe_layer call (route -> dispatch -> gate/up+SwiGLU ->
down -> combine) over one batch of synthetic tokens, with the weights, the
tokens and the router logits already resident in HBM.  Before every step
(warm-up and timed alike) a 1 GiB buffer is read end to end, so that no
expert weight is served from the L2 or the 256 MB Infinity Cache; that read
sits outside the timed events.  The flush reads rather than writes: a write
would leave up to 256 MB of dirty lines in the Infinity Cache, whose
write-back would then land inside the next timed step (about 55 us of extra
HBM traffic that the layer itself never causes).

The headline line is the DeepSeek-V3-shaped prefill layer at 4096 tokens
with Zipf-skewed routing (the metric's 4096-token point, the largest
workload that fits one GPU); the same JSON line carries the sweep over the
other workloads and token counts (Qwen3-30B-A3B- and DeepSeek-V3-shaped
decode at 1/8/32/128 tokens, the E4M3 layer at 32/128/512), the roofline of
the dominant kernel, and the C++ CPU oracle timed on this host at one thread
and at every thread of the host's share.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # dense, published
METRIC = "MoE-layer µs at 1/8/128/4096 tokens; achieved HBM GB/s & MFMA % of peak"
HEADLINE = ("dsv3_prefill", 4096)
DEFAULT_SWEEP = {"qwen3": (1, 8, 32, 128), "dsv3": (1, 8, 32, 128), "dsv3_prefill": (4096,),
                 "dsv3_fp8": (32, 128, 512)}
WORKLOAD_NAMES = {"qwen3": "qwen3-30b-a3b-moe-decode", "dsv3": "deepseek-v3-moe-decode",
                  "dsv3_fp8": "deepseek-v3-moe-decode-fp8", "dsv3_prefill": "deepseek-v3-moe-prefill-zipf",
                  "tiny": "tiny-moe-fp32"}
FLUSH_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (bytes and flops the method must move / compute)
# ---------------------------------------------------------------------------

_EB = {"f32": 4, "bf16": 2, "fp8": 1}


def layer_work(wl, T, touched):
    """Algorithmic HBM bytes and flops of one layer call.

    bytes: weights of the touched experts and of the shared expert, x and the
    router logits read, the dispatch payload written and read back by the
    GEMMs, the fp32 expert outputs (and shared output) written and read by
    the combine, and y written.  The SwiGLU activations between the two GEMMs
    are implementation traffic and are not counted."""
    d, F, Fs, k = wl.d_model, wl.d_ff, wl.d_ff_shared, wl.top_k
    wb, ab = _EB[wl.weight_dtype], _EB[wl.act_dtype]
    rb = 1 if wl.weight_dtype == "fp8" else ab  # dispatch payload element
    w = touched * 3 * d * F * wb + wl.num_shared * 3 * d * Fs * wb
    if wl.weight_dtype == "fp8":
        w += touched * 3 * (d // 128) * (F // 128) * 4 + wl.num_shared * 3 * (d // 128) * (Fs // 128) * 4
    act = T * d * ab + T * wl.num_experts * 4 + 2 * T * k * d * rb
    act += 2 * T * k * d * 4 + wl.num_shared * 2 * T * d * 4 + T * d * ab
    flops = 6 * d * F * T * k + 6 * d * Fs * T * wl.num_shared
    return w + act, flops, w


def gate_up_work(wl, T, touched):
    """Algorithmic bytes of one gate/up+SwiGLU launch: the gate and up weights
    of the touched experts (and the shared expert), the rows it reads, and the
    activations h it writes."""
    d, F, Fs, k = wl.d_model, wl.d_ff, wl.d_ff_shared, wl.top_k
    wb, ab = _EB[wl.weight_dtype], _EB[wl.act_dtype]
    rb = 1 if wl.weight_dtype == "fp8" else ab
    w = touched * 2 * F * d * wb + wl.num_shared * 2 * Fs * d * wb
    rows = T * k * d * rb + wl.num_shared * T * d * rb
    h = T * k * F * rb + wl.num_shared * T * Fs * rb
    flops = 4 * d * F * T * k + 4 * d * Fs * T * wl.num_shared
    return w + rows + h, flops


# ---------------------------------------------------------------------------
# device setup
# ---------------------------------------------------------------------------


class Layer:
    """Weights of one workload in HBM (every expert), generated in chunks."""

    def __init__(self, wl, seed=0, masked=False):
        import torch
        import moe_inputs as mi
        import combine_experts_amd as M
        self.wl = wl
        E, d, F, Fs = wl.num_experts, wl.d_model, wl.d_ff, wl.d_ff_shared
        self.cfg = M.make_config(wl.num_experts, wl.top_k, d, F, wl.num_shared, Fs, wl.n_group, wl.topk_group,
                                 wl.score, wl.weight, wl.routed_scale, wl.act_dtype, wl.weight_dtype,
                                 masked=masked)
        self.masked = masked
        fp8 = wl.weight_dtype == "fp8"
        tdt = {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8}[wl.weight_dtype]
        t0 = time.time()
        self.w13 = torch.empty((E, 2 * F, d), dtype=tdt, device="cuda")
        self.w2 = torch.empty((E, d, F), dtype=tdt, device="cuda")
        self.scales = []
        if fp8:
            self.w13s = torch.empty((E, 2 * F // 128, d // 128), device="cuda")
            self.w2s = torch.empty((E, d // 128, F // 128), device="cuda")
        per = max(1, (1 << 30) // (3 * d * F * _EB[wl.weight_dtype]))
        for e0 in range(0, E, per):
            n = min(per, E - e0)
            for name, dst, rows, cols, tid in (("w13", self.w13, 2 * F, d, mi.TID_W13),
                                               ("w2", self.w2, d, F, mi.TID_W2)):
                off = e0 * rows * cols
                if fp8:
                    c, s = mi.fp8_blocks(seed, tid, n * rows, cols, wl.w_std, offset=off)
                    dst[e0:e0 + n].copy_(torch.from_numpy(c).view(n, rows, cols))
                    sdst = self.w13s if name == "w13" else self.w2s
                    sdst[e0:e0 + n].copy_(torch.from_numpy(s).view(n, rows // 128, cols // 128))
                elif wl.weight_dtype == "bf16":
                    a = mi.normal_bf16(seed, tid, (n, rows, cols), wl.w_std, offset=off)
                    dst[e0:e0 + n].copy_(torch.from_numpy(a.view(np.int16)))
                else:
                    a = mi.normal_f32(seed, tid, (n, rows, cols), wl.w_std, offset=off)
                    dst[e0:e0 + n].copy_(torch.from_numpy(a))
            log(f"[bench] {wl.name}: experts {e0 + n}/{E} generated and uploaded ({time.time() - t0:.0f}s)")
        self.ws13 = self.ws2 = self.ws13s = self.ws2s = None
        if wl.num_shared:
            a = mi.gen_weight(wl, "ws13", 0, seed)
            b = mi.gen_weight(wl, "ws2", 0, seed)
            if fp8:
                self.ws13, self.ws13s = torch.from_numpy(a[0]).cuda(), torch.from_numpy(a[1]).cuda()
                self.ws2, self.ws2s = torch.from_numpy(b[0]).cuda(), torch.from_numpy(b[1]).cuda()
            else:
                conv = (lambda z: torch.from_numpy(z.view(np.int16))) if wl.weight_dtype == "bf16" else torch.from_numpy
                self.ws13, self.ws2 = conv(a).cuda(), conv(b).cuda()
        torch.cuda.synchronize()
        if fp8:
            self.W = M.make_weights(self.w13, self.w2, self.ws13, self.ws2, self.w13s, self.w2s, self.ws13s,
                                    self.ws2s)
        else:
            self.W = M.make_weights(self.w13, self.w2, self.ws13, self.ws2)
        log(f"[bench] {wl.name}: weights in HBM ({(self.w13.numel() + self.w2.numel()) * self.w13.element_size() / 1e9:.1f} GB) "
            f"in {time.time() - t0:.1f}s")


class Batch:
    def __init__(self, layer: Layer, wl, T, seed=0):
        """Tokens, logits and bias of workload wl (same shape and routing rule
        as the layer's) plus every buffer the layer call needs."""
        import torch
        import moe_inputs as mi
        import combine_experts_amd as M
        self.T = T
        x = mi.gen_x(wl, T, seed)
        self.x = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
        self.logits = torch.from_numpy(mi.gen_logits(wl, T, seed)).cuda()
        b = mi.gen_bias(wl, seed)
        self.bias = torch.from_numpy(b).cuda() if b is not None else None
        cfg = layer.cfg
        self.ws_bytes = M.moe_workspace_size(cfg, T)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device="cuda")
        ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16
        self.y = torch.empty((T, wl.d_model), dtype=ydt, device="cuda")
        # phase buffers for the per-kernel breakdown
        E, k, d = wl.num_experts, wl.top_k, wl.d_model
        self.idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        self.tw = torch.empty((T, k), device="cuda")
        self.count = torch.zeros(E, dtype=torch.int32, device="cuda")
        self.ticket = torch.empty((T, k), dtype=torch.int32, device="cuda")
        rows = M.moe_dispatch_rows(cfg, T)
        rb = 1 if wl.weight_dtype == "fp8" else _EB[wl.act_dtype]
        self.recv = torch.empty((rows, d * rb), dtype=torch.uint8, device="cuda")
        self.recv_scale = torch.empty((rows, d // 128), device="cuda") if wl.weight_dtype == "fp8" else None
        self.offset = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.row_of = torch.empty((T, k), dtype=torch.int32, device="cuda")
        routed = E * T if layer.masked else T * k
        self.eout = torch.empty((routed, d), device="cuda")
        self.sout = torch.empty((T, d), device="cuda") if wl.num_shared else None
        self.fws_bytes = M.moe_ffn_workspace_size(cfg, T)
        self.fws = torch.empty(max(self.fws_bytes, 256), dtype=torch.uint8, device="cuda")


def run_layer(layer, b):
    import combine_experts_amd as M
    M.moe_layer(layer.cfg, b.T, b.x, b.logits, b.bias, layer.W, b.y, b.ws, b.ws_bytes)


def run_phases(layer, b, marks):
    """The same layer through the separate entry points, with an event
    before every phase; marks: 6 recorded events."""
    import combine_experts_amd as M
    cfg, T = layer.cfg, b.T
    marks[0].record()
    if layer.masked:
        # one launch routes and writes the tokens; the GEMMs take the counters
        M.moe_route_dispatch(cfg, T, b.logits, b.bias, b.x, b.idx, b.tw, b.count, b.ticket, b.recv,
                             b.recv_scale, b.row_of)
        marks[1].record()
        groups = b.count
    else:
        M.moe_route(cfg, T, b.logits, b.bias, b.idx, b.tw, b.count, b.ticket)
        marks[1].record()
        M.moe_dispatch(cfg, T, b.x, b.idx, b.count, b.ticket, b.recv, b.recv_scale, b.offset, b.row_of)
        groups = b.offset
    marks[2].record()
    M.moe_ffn_gate_up(cfg, T, b.recv, b.recv_scale, groups, layer.W, b.x, b.fws, b.fws_bytes)
    marks[3].record()
    M.moe_ffn_down(cfg, T, groups, layer.W, b.fws, b.fws_bytes, b.eout, b.sout)
    marks[4].record()
    M.moe_combine(cfg, T, b.eout, b.row_of, b.tw, b.sout, b.y, b.count)
    marks[5].record()


def touched_experts(layer, b):
    """Experts with at least one row in this batch (read from the router's
    counters after one routing pass)."""
    import torch
    import combine_experts_amd as M
    M.moe_route(layer.cfg, b.T, b.logits, b.bias, b.idx, b.tw, b.count, b.ticket)
    torch.cuda.synchronize()
    c = b.count.cpu().numpy()
    b.count.zero_()
    torch.cuda.synchronize()
    return int((c > 0).sum()), c


def measure(layer, b, steps, warmup, flush, graph=False):
    import torch
    for _ in range(warmup):
        flush()
        run_layer(layer, b)
    torch.cuda.synchronize()
    step = lambda: run_layer(layer, b)  # noqa: E731
    if graph:
        # the same moe_layer call captured once and replayed (its launches
        # are fixed for a shape; the workspace counters return to zero)
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                run_layer(layer, b)
        torch.cuda.synchronize()
        step = g.replay
        for _ in range(warmup):
            flush()
            step()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        flush()
        s.record()
        step()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    layer_us = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])
    # per-phase breakdown through the separate entry points
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for m in marks:
        flush()
        run_phases(layer, b, m)
    torch.cuda.synchronize()
    ph = np.array([[m[i].elapsed_time(m[i + 1]) * 1e3 for i in range(5)] for m in marks])
    return layer_us, ph, wall


def measure_router(layer, b, wl, steps, flush):
    """Mean µs of the router GEMM (moe_router_logits_ws: logits = x W_r^T,
    fp32 out, its reduction split over workgroups where that helps) for the
    batch's tokens, caches flushed before every call.  Reported beside the
    layer, not inside it: the layer's input is the logits."""
    import torch
    import moe_inputs as mi
    import combine_experts_amd as M
    if wl.num_experts % 64:
        return None
    if getattr(layer, "w_router", None) is None:
        wr = mi.gen_router_weight(wl)
        layer.w_router = torch.from_numpy(wr.view(np.int16) if wr.dtype == np.uint16 else wr).cuda()
    out = torch.empty((b.T, wl.num_experts), dtype=torch.float32, device="cuda")
    nb = M.moe_router_workspace_size(layer.cfg, b.T)
    rws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")

    def call():
        M.moe_router_logits_ws(layer.cfg, b.T, b.x, layer.w_router, out, rws, nb)

    call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s_, e_ in ev:
        flush()
        s_.record()
        call()
        e_.record()
    torch.cuda.synchronize()
    return float(np.mean([s_.elapsed_time(e_) * 1e3 for s_, e_ in ev]))


def measure_fused(layer, b, wl, steps, warmup, flush):
    """Median us of moe_layer_fused (the whole layer in one persistent launch)
    from the logits, and from the hidden states (the launch computes the
    router logits itself), caches flushed before every call; None where the
    fused launch does not cover the shape."""
    import torch
    import moe_inputs as mi
    import combine_experts_amd as M
    if not M.moe_fused_supported(layer.cfg, b.T):
        return None
    nb = M.moe_fused_workspace_size(layer.cfg, b.T)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    if getattr(layer, "w_router", None) is None:
        wr = mi.gen_router_weight(wl)
        layer.w_router = torch.from_numpy(wr.view(np.int16) if wr.dtype == np.uint16 else wr).cuda()
    out = {}
    for key, lg, wr in (("fused_layer_us", b.logits, None), ("fused_from_hidden_us", None, layer.w_router)):
        call = lambda: M.moe_layer_fused(layer.cfg, b.T, b.x, lg, wr, b.bias, layer.W, b.y, ws, nb)  # noqa: E731
        for _ in range(warmup):
            flush()
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for s_, e_ in ev:
            flush()
            s_.record()
            call()
            e_.record()
        torch.cuda.synchronize()
        out[key] = round(float(np.median([s_.elapsed_time(e_) * 1e3 for s_, e_ in ev])), 2)
    if int(ws[16:20].view(torch.int32).item()) != 0:
        raise RuntimeError("moe_layer_fused: a grid-wide wait gave up (error word set)")
    return out


def host_threads():
    """Threads of this host's share: OMP_NUM_THREADS when set, else the CPUs
    this process may run on."""
    try:
        return max(1, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        return len(os.sched_getaffinity(0))


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family/model numbers
    (a virtualised host may print only the vendor's brand in the name)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                key, val = (s.strip() for s in line.split(":", 1))
                info.setdefault(key, val)
            elif info:
                break
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    nums = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(nums)})" if nums else name


def cpu_baseline(wl, T, threads, budget_s=10.0, seed=0):
    """The C++ oracle (oracle/moe_ref.cpp, as it stands) on the workload, on
    this host's cores with `threads` threads, in the metric's unit (us per
    layer call).

    Routing and dispatch of all T tokens are timed whole.  The expert FFNs are
    timed on a sample: touched experts taken at an even stride through the
    row-count order (so the sample spans hot and cold experts), enough of them
    for about budget_s seconds of work, and the shared expert on a
    proportional slice of the tokens; both are scaled to the whole layer by
    their FLOPs (the oracle's work is its multiply-adds: 6 d F per routed
    row).  The combine is timed on a slice of the tokens and scaled by token
    count.  Generating the sample experts' weights is input preparation and
    is not timed; the oracle reads them in their bf16 / E4M3 storage form."""
    import ctypes
    import moe_inputs as mi
    from oracle import moe_ref as R
    L = R.lib()
    E, k, d, F, Fs = wl.num_experts, wl.top_k, wl.d_model, wl.d_ff, wl.d_ff_shared
    fp8 = wl.weight_dtype == "fp8"
    c = R.config(wl, d_model=d, d_ff=F, d_ff_shared=Fs, act_dtype=wl.act_dtype, weight_dtype=wl.weight_dtype,
                 act_quant=fp8)
    x = np.ascontiguousarray(mi.gen_x(wl, T, seed))
    logits = np.ascontiguousarray(mi.gen_logits(wl, T, seed))
    bias = mi.gen_bias(wl, seed)
    bias = np.ascontiguousarray(bias) if bias is not None else None
    p = lambda a: a.ctypes.data if a is not None else None  # noqa: E731
    idx = np.empty((T, k), np.int32)
    tw = np.empty((T, k), np.float64)
    t0 = time.perf_counter()
    L.moe_ref_route(ctypes.byref(c), T, p(logits), p(bias), p(idx), p(tw))
    t_route = time.perf_counter() - t0
    counts, offsets = np.empty(E, np.int32), np.empty(E + 1, np.int32)
    row_of, tok = np.empty((T, k), np.int32), np.empty(T * k, np.int32)
    t0 = time.perf_counter()
    L.moe_ref_dispatch(ctypes.byref(c), T, p(idx), p(counts), p(offsets), p(row_of), p(tok))
    t_dispatch = time.perf_counter() - t0
    # sample experts: an even stride through the touched experts by row count
    rate = 4.5e9 * threads  # the oracle's FLOP/s per thread (measured), only to size the sample
    want = budget_s * rate * 0.8
    touched = sorted((int(counts[e]), e) for e in range(E) if counts[e] > 0)
    per_row = 6.0 * d * F
    total_rows = int(counts.sum())
    n_pick = 1
    while n_pick < len(touched) and per_row * total_rows * n_pick / len(touched) < want:
        n_pick += 1
    stride = len(touched) / n_pick
    sample = sorted({touched[int(stride * (i + 0.5))][1] for i in range(n_pick)})
    rows = int(sum(counts[e] for e in sample))
    # the sample's dispatched rows and weights (untimed preparation)
    sub_tok = np.concatenate([tok[offsets[e]:offsets[e + 1]] for e in sample]).astype(np.int32)
    # a compact weight array holding only the sample experts (sample expert i
    # in slot i), so that the whole layer's weights are never materialised
    ns = len(sample)
    cs = R.config(wl, d_model=d, d_ff=F, act_dtype=wl.act_dtype, weight_dtype=wl.weight_dtype, act_quant=fp8)
    cs.num_experts, cs.top_k, cs.n_group, cs.topk_group = ns, 1, 1, 1
    gw = [(mi.gen_weight(wl, "w13", e, seed), mi.gen_weight(wl, "w2", e, seed)) for e in sample]
    if fp8:
        a13 = np.ascontiguousarray(np.stack([g[0][0] for g in gw]))
        a2 = np.ascontiguousarray(np.stack([g[1][0] for g in gw]))
        s13 = np.ascontiguousarray(np.stack([g[0][1] for g in gw]))
        s2 = np.ascontiguousarray(np.stack([g[1][1] for g in gw]))
        W = R.RefWeights(p(a13), p(a2), None, None, p(s13), p(s2), None, None)
    else:
        a13 = np.ascontiguousarray(np.stack([g[0] for g in gw]))
        a2 = np.ascontiguousarray(np.stack([g[1] for g in gw]))
        W = R.RefWeights(p(a13), p(a2), None, None, None, None, None, None)
    comp_off = np.zeros(ns + 1, np.int32)
    for i, e in enumerate(sample):
        comp_off[i + 1] = comp_off[i] + counts[e]
    recv = np.empty((rows, d), np.float64)
    eout = np.empty((rows, d), np.float64)
    cg = R.config(wl, d_model=d, d_ff=F, act_dtype=wl.act_dtype, weight_dtype=wl.weight_dtype)
    cg.top_k = 1
    t0 = time.perf_counter()
    L.moe_ref_gather(ctypes.byref(cg), rows, p(x), p(sub_tok), p(recv))
    L.moe_ref_expert_ffn(ctypes.byref(cs), rows, p(recv), p(comp_off), ctypes.byref(W), None, p(eout), None, threads)
    t_ffn = time.perf_counter() - t0
    # shared expert on a proportional slice of the tokens
    t_shared, Ts = 0.0, 0
    if wl.num_shared:
        Ts = max(1, int(round(T * n_pick / len(touched))))
        a, b = mi.gen_weight(wl, "ws13", 0, seed), mi.gen_weight(wl, "ws2", 0, seed)
        ch = R.config(wl, d_model=d, d_ff=Fs, act_dtype=wl.act_dtype, weight_dtype=wl.weight_dtype, act_quant=fp8)
        ch.num_experts, ch.top_k, ch.n_group, ch.topk_group = 1, 1, 1, 1
        keep = (np.ascontiguousarray(a[0] if fp8 else a), np.ascontiguousarray(b[0] if fp8 else b))
        ks = (np.ascontiguousarray(a[1]), np.ascontiguousarray(b[1])) if fp8 else (None, None)
        WS = R.RefWeights(p(keep[0]), p(keep[1]), None, None, p(ks[0]), p(ks[1]), None, None)
        xs = np.ascontiguousarray(R._f64(mi.bf16_bits_to_f32(x[:Ts]) if x.dtype == np.uint16 else x[:Ts]))
        so = np.empty((Ts, d), np.float64)
        t0 = time.perf_counter()
        L.moe_ref_expert_ffn(ctypes.byref(ch), Ts, p(xs), p(np.array([0, Ts], np.int32)), ctypes.byref(WS), None,
                             p(so), None, threads)
        t_shared = time.perf_counter() - t0
    # combine on a slice of the tokens (their rows taken from the sample output)
    Tc = min(T, 256)
    fake = np.ascontiguousarray(np.resize(eout, (Tc * k, d)))
    rc = np.ascontiguousarray(np.arange(Tc * k, dtype=np.int32).reshape(Tc, k))
    yc = np.empty((Tc, d), np.float64)
    t0 = time.perf_counter()
    L.moe_ref_combine(ctypes.byref(c), Tc, p(fake), p(rc), p(np.ascontiguousarray(tw[:Tc])), None, p(yc))
    t_combine = time.perf_counter() - t0
    routed_scale_up = total_rows / rows
    est = (t_route + t_dispatch + t_ffn * routed_scale_up + (t_shared * T / Ts if Ts else 0.0)
           + t_combine * T / Tc)
    return {"value": round(est * 1e6, 1), "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": (f"C++ oracle (double accumulation, {threads} thread{'s' if threads > 1 else ''}) on the "
                       f"{WORKLOAD_NAMES[wl.name]} layer at {T} tokens: route and dispatch of all tokens timed "
                       f"whole ({(t_route + t_dispatch) * 1e3:.1f} ms); expert FFNs timed on {ns} of "
                       f"{len(touched)} touched experts ({rows} of {total_rows} routed rows, "
                       f"{t_ffn:.2f} s) and scaled by rows; shared expert on {Ts} of {T} tokens "
                       f"({t_shared:.2f} s) and combine on {Tc} tokens ({t_combine * 1e3:.1f} ms), scaled by "
                       f"tokens; weight generation untimed"),
            "timed_s": round(t_route + t_dispatch + t_ffn + t_shared + t_combine, 2)}


def _code_only(text):
    """Source text without its // and /* */ comments (string literals in
    these sources hold no comment markers), blank lines and the spaces that
    begin or end a line, so that editing a comment or the layout does not
    change a kernel's key."""
    text = re.sub(rb"/\*.*?\*/", b"", text, flags=re.S)
    text = re.sub(rb"//[^\n]*", b"", text)
    return b"\n".join(line.strip() for line in text.splitlines() if line.strip())


def source_digest(source):
    """First 16 hex digits of the SHA-256 of a kernel source file followed by
    every local header it includes, transitively, each once in include order
    (looked up in csrc/, then include/), comments removed."""
    dirs = [os.path.join(ROOT, "combine_experts_amd", "csrc"), os.path.join(ROOT, "include")]
    h, seen = hashlib.sha256(), set()

    def add(name):
        if name in seen:
            return
        seen.add(name)
        path = next((os.path.join(d, name) for d in dirs if os.path.exists(os.path.join(d, name))), None)
        if path is None:
            return
        text = open(path, "rb").read()
        h.update(_code_only(text))
        for inc in re.findall(rb'^\s*#\s*include\s+"([^"]+)"', text, re.M):
            add(inc.decode())

    add(source)
    return h.hexdigest()[:16]


def kernel_traffic(key, source):
    """HBM bytes per launch measured with rocprofv3 counters, from the
    committed summary, if it was taken on the current kernel source and the
    headers it includes."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.md")
    if not os.path.exists(path):
        return None
    digest = source_digest(source)
    for line in open(path):
        m = re.match(r"\|\s*" + re.escape(key) + r"\s*\|\s*([0-9a-f]{16})\s*\|\s*([0-9.eE+,]+)\s*\|", line)
        if m and m.group(1) == digest:
            return float(m.group(2).replace(",", ""))
    return None


def uses_tiled(wl, T):
    """The library's choice of grouped-GEMM kernel: the LDS-tiled one for
    bf16 batches with at least 5 (d_model >= 6144), 8 (d_model >= 3072) or
    12 rows per expert on average, else the weight-streaming one."""
    r = 5 if wl.d_model >= 6144 else 8 if wl.d_model >= 3072 else 12
    return wl.weight_dtype == "bf16" and T * wl.top_k >= r * wl.num_experts


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=",".join(DEFAULT_SWEEP),
                    help="comma list of workloads (qwen3,dsv3,dsv3_prefill,dsv3_fp8,tiny)")
    ap.add_argument("--tokens", default=None, help="override the token counts, e.g. 1,8,128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--no-router", action="store_true",
                    help="skip timing the router GEMM (its prefill-sized launches use the same tiled kernel "
                         "as the down pass, which would mix the two in a profile)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of moe_layer captured in a HIP graph instead of direct calls")
    ap.add_argument("--layout", choices=("auto", "compact", "masked"), default="auto",
                    help="dispatch layout: auto (masked for bf16 layers at 8 tokens or fewer, compact "
                         "otherwise), compact (T*k rows from a scan of the counters) or masked "
                         "(E*T rows, route and dispatch in one launch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (a plain copy of known size for "
                         "scaling the profiler's byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import combine_experts_amd  # noqa: F401  (fails loudly if the HIP library is missing)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB three times (1048576 KiB read and written per copy)")
        return
    flush_buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def flush():
        if args.no_flush:
            return
        flush_buf.sum()  # reads 1 GiB; the one-element result is dropped

    names = [n for n in args.workloads.split(",") if n]
    sweep = []
    headline = None
    layers = {}
    order = [n for n in ("qwen3", "tiny", "dsv3", "dsv3_prefill", "dsv3_fp8") if n in names]
    for name in order:
        wl = mi.WORKLOADS[name]
        key = "dsv3" if name == "dsv3_prefill" else name
        if key not in layers:
            for k_ in list(layers):
                if k_ != key:
                    del layers[k_]
            torch.cuda.empty_cache()
            layers[key] = Layer(wl, masked=args.layout == "masked")
        layer = layers[key]  # the prefill workload reuses the decode weights; only the bias differs
        toks = DEFAULT_SWEEP.get(name, wl.tokens)
        if args.tokens:
            toks = tuple(int(t) for t in args.tokens.split(","))
        for T in toks:
            # auto: the masked layout (route and dispatch in one launch) where
            # it measured faster, at bf16 decode of 8 tokens or fewer (Qwen3
            # shapes 1 token 42.1 -> 38.2 us, 8 tokens 101.6 -> 98.3 us; at 128
            # tokens compact is faster, 233 against 240 us)
            if args.layout == "auto":
                layer.masked = T <= 8 and wl.weight_dtype == "bf16"
                layer.cfg.masked_layout = 1 if layer.masked else 0
            b = Batch(layer, wl, T)
            b_wl = wl
            D, counts = touched_experts(layer, b)
            layer_us, ph, wall = measure(layer, b, args.steps, args.warmup, flush, graph=args.graph)
            nbytes, flops, wbytes = layer_work(b_wl, T, D)
            med = float(np.median(layer_us))
            gu_bytes, gu_flops = gate_up_work(b_wl, T, D)
            gu_us = float(ph[:, 2].mean())
            peak_t = MFMA_PEAK_TFLOPS[b_wl.weight_dtype]
            ent = {
                "workload": WORKLOAD_NAMES[name], "tokens": T, "layout": "masked" if layer.masked else "compact",
                "launch": "hip graph replay" if args.graph else "direct", "touched_experts": D,
                "grouped_gemm": "lds_tiled" if uses_tiled(b_wl, T) else "weight_streaming",
                "layer_us_median": round(med, 2), "layer_us_p10": round(float(np.percentile(layer_us, 10)), 2),
                "layer_us_p90": round(float(np.percentile(layer_us, 90)), 2),
                "tokens_per_s": round(T / med * 1e6, 1),
                "alg_bytes": nbytes, "alg_flops": flops,
                "hbm_GBps": round(nbytes / med / 1e3, 1),
                "hbm_frac": round(nbytes / med / 1e3 / HBM_PEAK_GBS, 4),
                "tflops": round(flops / med / 1e6, 2),
                "mfma_frac": round(flops / med / 1e6 / peak_t, 5),
                "hbm_roof_us": round(nbytes / HBM_PEAK_GBS / 1e3, 2),
                "mfma_roof_us": round(flops / peak_t / 1e6, 2),
                # the binding roof is the larger of the two; frac = roof / measured
                "binding_roof": "hbm" if nbytes / HBM_PEAK_GBS / 1e3 >= flops / peak_t / 1e6 else "mfma",
                "binding_frac": round(max(nbytes / HBM_PEAK_GBS / 1e3, flops / peak_t / 1e6) / med, 4),
                "phase_us_mean": {p: round(float(v), 2) for p, v in
                                  zip(("route", "dispatch", "gate_up", "down", "combine"), ph.mean(axis=0))},
                "gate_up_GBps": round(gu_bytes / gu_us / 1e3, 1),
                "max_expert_share": round(float(counts.max() / counts.sum()), 4),
                "empty_experts": int((counts == 0).sum()),
                "imbalance_factor_8_ranks": round(float(counts.reshape(8, -1).sum(1).max()
                                                        / counts.reshape(8, -1).sum(1).mean()), 3)
                if wl.num_experts % 8 == 0 else None,
            }
            rg_us = None if args.no_router else measure_router(layer, b, b_wl, args.steps, flush)
            if rg_us is not None:
                ab = _EB[b_wl.act_dtype]
                rg_bytes = b_wl.num_experts * b_wl.d_model * ab + T * b_wl.d_model * ab + T * b_wl.num_experts * 4
                ent["router_gemm_us"] = round(rg_us, 2)
                ent["router_gemm_GBps"] = round(rg_bytes / rg_us / 1e3, 1)
            fz = measure_fused(layer, b, b_wl, args.steps, args.warmup, flush)
            if fz is not None:
                ent.update(fz)
                if "router_gemm_us" in ent:
                    ent["router_gemm_plus_layer_us"] = round(ent["router_gemm_us"] + med, 2)
            sweep.append(ent)
            log(f"[bench] {name} T={T}: layer {med:.1f} us (HBM {ent['hbm_frac'] * 100:.1f}% of peak, "
                f"roof {ent['hbm_roof_us']:.1f} us), phases {ent['phase_us_mean']}"
                + (f", router GEMM {ent['router_gemm_us']} us" if "router_gemm_us" in ent else "")
                + (f", fused {ent['fused_layer_us']} us ({ent['fused_from_hidden_us']} us from hidden states)"
                   if "fused_layer_us" in ent else ""))
            if (name, T) == HEADLINE:
                headline = (ent, layer_us, wall, gu_bytes, gu_flops, gu_us, b_wl)
            del b
            torch.cuda.empty_cache()
    layers.clear()

    if headline is None:
        ent, layer_us, wall, gu_bytes, gu_flops, gu_us, hwl = (sweep[-1], None, None, None, None, None, None)
    else:
        ent, layer_us, wall, gu_bytes, gu_flops, gu_us, hwl = headline
    out = {
        "metric": METRIC,
        "value": ent["layer_us_median"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ent["layer_us_median"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shapes; random weights)",
        "config": {"workload": ent["workload"], "tokens": ent["tokens"], "layout": ent["layout"],
                   "launch": ent["launch"],
                   "cache": "cold (1 GiB read before each step)"},
    }
    if gu_us:
        tiled = uses_tiled(hwl, ent["tokens"])
        kname = ("gemm_tiled_kernel<true, 256> gate/up+SwiGLU (moe_ffn_gate_up)" if tiled
                 else "ffn_kernel gate/up+SwiGLU (moe_ffn_gate_up)")
        out["roofline"] = {"kernel": kname, "bound": "hbm",
                           "achieved": round(gu_bytes / gu_us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gu_bytes / gu_us / 1e3 / HBM_PEAK_GBS, 4),
                           "traffic": kernel_traffic(f"gate_up {ent['workload']} T={ent['tokens']}",
                                                     "gemm_tiled.hip" if tiled else "ffn.hip"),
                           "alg_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 2),
                           "alg_flops_per_launch": gu_flops,
                           "mfma_frac": round(gu_flops / gu_us / 1e6 / MFMA_PEAK_TFLOPS[hwl.weight_dtype], 4)}
    if not args.no_cpu_baseline and headline is not None:
        nt = host_threads()
        log(f"[bench] timing the C++ CPU oracle on the headline workload ({nt} threads, then 1)")
        cb = cpu_baseline(hwl, ent["tokens"], nt)
        one = cpu_baseline(hwl, ent["tokens"], 1)
        cb["cpu_model"] = cpu_model()
        cb["single_thread"] = {"value": one["value"], "unit": "us", "cores": 1, "sample": one["sample"],
                               "timed_s": one["timed_s"]}
        out["cpu_baseline"] = cb
    out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
