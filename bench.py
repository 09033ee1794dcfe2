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

The headline line is the Qwen3-30B-A3B-shaped decode layer at 128 tokens;
the same JSON line carries the sweep over the other workloads and token
counts (DeepSeek-V3-shaped decode in bf16 and E4M3, and the 4096-token
prefill with Zipf-skewed routing), the roofline of the dominant kernel, and
the CPU oracle timed on this host.

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
HEADLINE = ("qwen3", 128)
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
    """Mean µs of the router GEMM (moe_router_logits: logits = x W_r^T, fp32
    out) for the batch's tokens, caches flushed before every call.  Reported
    beside the layer, not inside it: the layer's input is the logits."""
    import torch
    import moe_inputs as mi
    import combine_experts_amd as M
    if wl.num_experts % 64:
        return None
    if getattr(layer, "w_router", None) is None:
        wr = mi.gen_router_weight(wl)
        layer.w_router = torch.from_numpy(wr.view(np.int16) if wr.dtype == np.uint16 else wr).cuda()
    out = torch.empty((b.T, wl.num_experts), dtype=torch.float32, device="cuda")
    M.moe_router_logits(layer.cfg, b.T, b.x, layer.w_router, out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s_, e_ in ev:
        flush()
        s_.record()
        M.moe_router_logits(layer.cfg, b.T, b.x, layer.w_router, out)
        e_.record()
    torch.cuda.synchronize()
    return float(np.mean([s_.elapsed_time(e_) * 1e3 for s_, e_ in ev]))


def cpu_baseline(wl, T, seed=0):
    """The oracle, as it stands, on the headline workload: the whole layer
    for T tokens, all weights read from the generator's bf16 values."""
    import moe_inputs as mi
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    x = mi.bf16_bits_to_f32(mi.gen_x(wl, T, seed)).astype(np.float64)
    logits = mi.gen_logits(wl, T, seed)
    bias = mi.gen_bias(wl, seed)

    def get_expert(e):
        a = mi.bf16_bits_to_f32(mi.gen_weight(wl, "w13", e, seed)).astype(np.float64)
        b = mi.bf16_bits_to_f32(mi.gen_weight(wl, "w2", e, seed)).astype(np.float64)
        return a, b
    # weight generation is input preparation: fetch every expert first
    idx, _, _ = O.route(logits, bias, wl)
    cache = {int(e): get_expert(int(e)) for e in np.unique(idx)}
    # repeat for about ten seconds (at least 3 runs) and report the median
    runs = []
    t_start = time.perf_counter()
    while len(runs) < 3 or (time.perf_counter() - t_start < 10.0 and len(runs) < 1000):
        t0 = time.perf_counter()
        O.layer(x, logits, bias, wl, lambda e: cache[e])
        runs.append(time.perf_counter() - t0)
    return {"value": round(float(np.median(runs)) * 1e6, 1), "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": f"whole {WORKLOAD_NAMES[wl.name]} layer at {T} tokens (float64 numpy oracle: route, "
                      f"dispatch, {len(cache)} experts, combine), median of {len(runs)} runs over "
                      f"{time.perf_counter() - t_start:.1f} s, weight decode excluded"}


def kernel_traffic(key):
    """HBM bytes per launch measured with rocprofv3 counters, from the
    committed summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.md")
    if not os.path.exists(path):
        return None
    src = open(os.path.join(ROOT, "combine_experts_amd", "csrc", "ffn.hip"), "rb").read()
    digest = hashlib.sha256(src).hexdigest()[:16]
    for line in open(path):
        m = re.match(r"\|\s*" + re.escape(key) + r"\s*\|\s*([0-9a-f]{16})\s*\|\s*([0-9.eE+]+)\s*\|", line)
        if m and m.group(1) == digest:
            return float(m.group(2))
    return None


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
            sweep.append(ent)
            log(f"[bench] {name} T={T}: layer {med:.1f} us (HBM {ent['hbm_frac'] * 100:.1f}% of peak, "
                f"roof {ent['hbm_roof_us']:.1f} us), phases {ent['phase_us_mean']}"
                + (f", router GEMM {ent['router_gemm_us']} us" if "router_gemm_us" in ent else ""))
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
        out["roofline"] = {"kernel": "ffn_kernel gate/up+SwiGLU (moe_ffn_gate_up)", "bound": "hbm",
                           "achieved": round(gu_bytes / gu_us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gu_bytes / gu_us / 1e3 / HBM_PEAK_GBS, 4),
                           "traffic": kernel_traffic(f"gate_up {ent['workload']} T={ent['tokens']}"),
                           "alg_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 2)}
    if not args.no_cpu_baseline and headline is not None:
        log("[bench] timing the CPU oracle on the headline workload")
        out["cpu_baseline"] = cpu_baseline(hwl, ent["tokens"])
    out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
