"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
entry-point chain through the C ABI, and the oracle-side checks.

Inputs come from moe_inputs; expected values only from oracle/.  Nothing here
feeds a GPU result back into the oracle except the routing choice, and only
where the oracle itself reports a near-tie."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import moe_inputs as mi
from oracle import moe_oracle as O
from oracle import moe_ref as R

# max |err| / max |ref| bounds per weight dtype: bf16 and fp8 as the layer's
# accuracy target states, against the float64 oracle with exact activations
# (E4M3 weights are their code * scale values); fp32 from the arithmetic (fp32
# accumulation over K <= 2048 terms of O(1) products keeps relative errors
# near 1e-6).
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
# E4M3 layers are also compared with the oracle's quantised-activation form
# (x and h rounded to E4M3 per 1x128 block, as the kernels do).  Layer
# outputs: a tighter bound.  One expert's outputs: the h codes are decided on
# fp32 values whose accumulation order differs between kernel and oracle, so
# a few codes flip by one E4M3 step (6.25-12.5% of that element), which moved
# a one-row expert by 2.3e-2 (1024 experts, d_ff 256); a wrong tile or scale
# moves it by far more than the 6e-2 bar.
TOL_FP8_QUANT_FORM = {"layer": 2e-2, "expert": 6e-2}
# a routing choice may differ only where the oracle's deciding keys are this close
TIE = 1e-5

_TORCH_DT = {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8}
_ES = {"f32": 4, "bf16": 2, "fp8": 1}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def x_values(wl, x_host) -> np.ndarray:
    """float64 values of the token activations."""
    if wl.act_dtype == "f32":
        return x_host.astype(np.float64)
    return mi.bf16_bits_to_f32(x_host).astype(np.float64)


def cfg_of(wl):
    import combine_experts_amd as M
    return M.make_config(wl.num_experts, wl.top_k, wl.d_model, wl.d_ff, wl.num_shared, wl.d_ff_shared,
                         wl.n_group, wl.topk_group, wl.score, wl.weight, wl.routed_scale, wl.act_dtype,
                         wl.weight_dtype)


class Weights:
    """Device copy of a workload's expert weights.  Experts outside `experts`
    are filled with NaN (NaN codes and scales for E4M3), so any read of an
    untouched expert would poison the outputs."""

    def __init__(self, wl, experts=None, seed=0):
        self.wl, self.seed = wl, seed
        E, d, F, Fs = wl.num_experts, wl.d_model, wl.d_ff, wl.d_ff_shared
        wdt = wl.weight_dtype
        tdt = _TORCH_DT[wdt]
        nan = {"f32": float("nan"), "bf16": 0x7FC0, "fp8": 0x7F}[wdt]
        self.experts = sorted(set(range(E) if experts is None else experts))
        self.w13 = torch.full((E, 2 * F, d), nan, dtype=tdt, device="cuda")
        self.w2 = torch.full((E, d, F), nan, dtype=tdt, device="cuda")
        self.fp8 = wdt == "fp8"
        if self.fp8:
            self.w13s = torch.full((E, 2 * F // 128, d // 128), float("nan"), device="cuda")
            self.w2s = torch.full((E, d // 128, F // 128), float("nan"), device="cuda")
        self.host = {}
        for e in self.experts:
            self._fill(e)
        self.ws13 = self.ws2 = self.ws13s = self.ws2s = None
        if wl.num_shared:
            a = mi.gen_weight(wl, "ws13", 0, seed)
            b = mi.gen_weight(wl, "ws2", 0, seed)
            self.host["shared"] = (a, b)
            if self.fp8:
                self.ws13, self.ws13s = dev(a[0]), dev(a[1])
                self.ws2, self.ws2s = dev(b[0]), dev(b[1])
            else:
                self.ws13, self.ws2 = dev(a), dev(b)
        torch.cuda.synchronize()

    def _fill(self, e):
        a = mi.gen_weight(self.wl, "w13", e, self.seed)
        b = mi.gen_weight(self.wl, "w2", e, self.seed)
        self.host[e] = (a, b)
        if self.fp8:
            self.w13[e].copy_(dev(a[0]))
            self.w13s[e].copy_(dev(a[1]))
            self.w2[e].copy_(dev(b[0]))
            self.w2s[e].copy_(dev(b[1]))
        else:
            self.w13[e].copy_(dev(a))
            self.w2[e].copy_(dev(b))

    def ensure(self, experts):
        new = [e for e in set(int(v) for v in experts) if e not in self.host]
        for e in new:
            self._fill(e)
        if new:
            torch.cuda.synchronize()

    def moe_weights(self):
        import combine_experts_amd as M
        if self.fp8:
            return M.make_weights(self.w13, self.w2, self.ws13, self.ws2, self.w13s, self.w2s, self.ws13s,
                                  self.ws2s)
        return M.make_weights(self.w13, self.w2, self.ws13, self.ws2)

    def _f64(self, m):
        if self.fp8:
            return O.dequant_blocks(m[0], m[1])
        if self.wl.weight_dtype == "bf16":
            return mi.bf16_bits_to_f32(m).astype(np.float64)
        return m.astype(np.float64)

    @functools.lru_cache(maxsize=24)
    def get_expert(self, e):
        a, b = self.host[e]
        return self._f64(a), self._f64(b)

    @functools.lru_cache(maxsize=1)
    def get_shared(self):
        a, b = self.host["shared"]
        return self._f64(a), self._f64(b)


class Inputs:
    def __init__(self, wl, T, seed=0):
        self.wl, self.T = wl, T
        self.x_host = mi.gen_x(wl, T, seed)
        self.logits = mi.gen_logits(wl, T, seed)
        self.bias = mi.gen_bias(wl, seed)
        self.x = dev(self.x_host)
        self.logits_d = dev(self.logits)
        self.bias_d = dev(self.bias) if self.bias is not None else None
        self.xv = x_values(wl, self.x_host)


def run_chain(wl, inp: Inputs, W: Weights | None, stages=("route", "dispatch", "ffn", "combine"),
              pad_rows=16):
    """Run the entry points in order; returns host copies of every output."""
    import combine_experts_amd as M
    cfg = cfg_of(wl)
    T, E, k, d = inp.T, wl.num_experts, wl.top_k, wl.d_model
    out = {}
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    tw = torch.full((T, k), float("nan"), device="cuda")
    count = torch.zeros(E, dtype=torch.int32, device="cuda")
    ticket = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    M.moe_route(cfg, T, inp.logits_d, inp.bias_d, idx, tw, count, ticket)
    torch.cuda.synchronize()
    out.update(idx=host(idx), w=host(tw), count=host(count), ticket=host(ticket))
    if "dispatch" not in stages:
        return out
    rows = M.moe_dispatch_rows(cfg, T)
    rdt = "fp8" if wl.weight_dtype == "fp8" else wl.act_dtype
    # sentinel-filled receive buffer with spare rows past the end
    recv = torch.full((rows + pad_rows, d * _ES[rdt]), 0x7F, dtype=torch.uint8, device="cuda")
    recv_scale = (torch.full((rows + pad_rows, d // 128), float("nan"), device="cuda")
                  if wl.weight_dtype == "fp8" else None)
    offset = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    row_of = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    M.moe_dispatch(cfg, T, inp.x, idx, count, ticket, recv, recv_scale, offset, row_of)
    torch.cuda.synchronize()
    out.update(recv=host(recv), offset=host(offset), row_of=host(row_of), rows=rows)
    if recv_scale is not None:
        out["recv_scale"] = host(recv_scale)
    if "ffn" not in stages:
        return out
    eout = torch.full((T * k, d), float("nan"), device="cuda")
    sout = torch.full((T, d), float("nan"), device="cuda") if wl.num_shared else None
    nbytes = M.moe_ffn_workspace_size(cfg, T)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    M.moe_expert_ffn(cfg, T, recv, recv_scale, offset, W.moe_weights(), inp.x, eout, sout, ws, nbytes)
    torch.cuda.synchronize()
    out["eout"] = host(eout)
    if sout is not None:
        out["sout"] = host(sout)
    if "combine" not in stages:
        return out
    ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16
    y = torch.empty((T, d), dtype=ydt, device="cuda")
    M.moe_combine(cfg, T, eout, row_of, tw, sout, y, count)
    torch.cuda.synchronize()
    out["y"] = host(y)
    out["count_after"] = host(count)
    return out


def y_values(wl, y):
    return y.astype(np.float64) if wl.act_dtype == "f32" else mi.bf16_bits_to_f32(y).astype(np.float64)


# ---------------------------------------------------------------------------
# checks
# ---------------------------------------------------------------------------


def check_near_tie_choice(wl, keys, gscores, sel, sel_ref):
    """A selection that differs from the oracle's at a near-tie must still be
    a valid group-limited top-k up to the tie band: at most topk_group groups,
    each scoring within TIE of the oracle's topk_group-th group score; inside
    the selected experts' groups no unselected key above the smallest selected
    key by more than TIE; and, where the groups agree with the oracle's, every
    swapped-in or swapped-out key within TIE of the oracle's k-th key."""
    E, k, G, kg = wl.num_experts, wl.top_k, wl.n_group, wl.topk_group
    sel = np.asarray(sel)
    assert len(set(sel.tolist())) == k and ((sel >= 0) & (sel < E)).all(), sel
    keys = keys.astype(np.float64)
    gsz = E // G
    groups = set((sel // gsz).tolist())
    ref_groups = set((np.asarray(sel_ref) // gsz).tolist())
    if G > 1:
        g = gscores.astype(np.float64)
        kth_g = np.sort(g)[::-1][kg - 1]
        assert len(groups) <= kg, (groups, kg)
        assert all(g[q] >= kth_g - TIE for q in groups), (g, groups)
    elig = np.array([e // gsz in groups for e in range(E)])
    unsel = elig.copy()
    unsel[sel] = False
    if unsel.any():
        assert keys[unsel].max() <= keys[sel].min() + TIE, "selection is not a top-k within its groups"
    if groups <= ref_groups or G == 1:
        kth = np.sort(keys[np.asarray(sel_ref)])[0]
        for e in set(sel.tolist()) ^ set(np.asarray(sel_ref).tolist()):
            assert abs(keys[e] - kth) <= TIE, (e, keys[e], kth)


def check_route(wl, inp: Inputs, r):
    """Indices bit-exact except near-ties; weights close; counts = bincount;
    tickets of each expert a permutation of 0..count-1.  Returns the mask of
    tokens whose routing legitimately differs."""
    T, E, k = inp.T, wl.num_experts, wl.top_k
    idx_ref, w_ref, info = O.route(inp.logits, inp.bias, wl)
    idx = r["idx"]
    diff = (idx != idx_ref).any(axis=1)
    if diff.any():
        margin = O.routing_margins(info, wl)
        bad = diff & ~(margin <= TIE)
        assert not bad.any(), f"routing differs beyond near-ties at tokens {np.nonzero(bad)[0][:8]}"
        gs = info["group_scores"]
        for t in np.nonzero(diff)[0]:
            check_near_tie_choice(wl, info["keys"][t], gs[t] if gs is not None else None, idx[t], idx_ref[t])
    same = ~diff
    assert np.allclose(r["w"][same], w_ref[same], rtol=2e-5, atol=1e-6), \
        np.abs(r["w"][same] - w_ref[same]).max()
    assert np.array_equal(r["count"], np.bincount(idx.reshape(-1), minlength=E))
    for e in range(E):
        tk = np.sort(r["ticket"][idx == e])
        assert np.array_equal(tk, np.arange(r["count"][e])), e
    return diff


def check_dispatch(wl, inp: Inputs, r):
    """Canonical (token-ordered) layout bit-exact; every row written once;
    payload bytes equal x (or its E4M3 codes and scales)."""
    T, E, k, d = inp.T, wl.num_experts, wl.top_k, wl.d_model
    idx = r["idx"]
    counts, offsets, row_of_ref, tok_ref = O.dispatch(idx, E)
    assert np.array_equal(r["offset"], offsets)
    row_of = r["row_of"]
    assert np.array_equal(row_of, r["offset"][idx] + r["ticket"])
    assert sorted(row_of.reshape(-1).tolist()) == list(range(T * k))
    tok = np.empty(T * k, dtype=np.int64)
    tok[row_of.reshape(-1)] = np.repeat(np.arange(T), k)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        assert np.array_equal(np.sort(tok[lo:hi]), tok_ref[lo:hi]), e
    recv = r["recv"]
    if wl.weight_dtype == "fp8":
        x32 = inp.xv.astype(np.float32)
        codes, scales = O.quantize_rows_1x128(x32)
        assert np.array_equal(recv[:T * k], codes[tok]), "E4M3 codes differ"
        assert np.array_equal(r["recv_scale"][:T * k], scales[tok]), "E4M3 scales differ"
        if wl.num_shared:
            assert np.array_equal(recv[T * k:T * k + T], codes)
            assert np.array_equal(r["recv_scale"][T * k:T * k + T], scales)
        assert (recv[r["rows"]:] == 0x7F).all()
    else:
        xb = np.ascontiguousarray(inp.x_host).view(np.uint8).reshape(T, -1)
        assert np.array_equal(recv[:T * k], xb[tok])
        assert (recv[T * k:] == 0x7F).all()
    return tok


def rel_err(got, ref):
    m = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (m if m > 0 else 1.0))


def sample(n, want, rng):
    if n <= want:
        return np.arange(n)
    pick = set([0, n - 1]) | set(rng.choice(n, size=want - 2, replace=False).tolist())
    return np.array(sorted(pick))


def _check_rows(wl, got, ref_of, what, layer=False):
    """got against the oracle; ref_of(q) gives the oracle's rows for
    act_quant = q.  bf16 and fp32: exact activations, TOL.  E4M3: the
    quantised-activation form within TOL_FP8_QUANT_FORM; layer outputs also
    against exact activations within TOL (the layer's fp8 bar).  An
    expert's own output is not held to TOL against exact activations: E4M3
    rounding of its input rows alone moves it by up to ~6% (an expert sums no
    errors from other experts, unlike the layer).  Returns the error against
    exact activations."""
    err = rel_err(got, ref_of(False))
    if wl.weight_dtype != "fp8":
        assert err <= TOL[wl.weight_dtype], (what, err)
        return err
    errq = rel_err(got, ref_of(True))
    assert errq <= TOL_FP8_QUANT_FORM["layer" if layer else "expert"], (what, "quantised form", errq)
    if layer:
        assert err <= TOL["fp8"], (what, "exact activations", err)
    return err


def check_ffn(wl, inp: Inputs, r, W: Weights, tok, max_experts=None, rng=None):
    """Expert outputs of whole experts (all, or a sample) against the oracle's
    SwiGLU expert on the same rows; shared expert on sampled tokens."""
    rng = rng or np.random.default_rng(0)
    E = wl.num_experts
    off = r["offset"]
    active = [e for e in range(E) if off[e + 1] > off[e]]
    if max_experts is not None and len(active) > max_experts:
        big = max(active, key=lambda e: off[e + 1] - off[e])
        pick = set(rng.choice(active, size=max_experts - 1, replace=False).tolist()) | {big}
        active = sorted(pick)
    worst = 0.0
    for e in active:
        lo, hi = off[e], off[e + 1]
        err = _check_rows(wl, r["eout"][lo:hi],
                          lambda q: O.swiglu_expert(inp.xv[tok[lo:hi]], *W.get_expert(e), act_quant=q), e)
        worst = max(worst, err)
    if wl.num_shared:
        ts = sample(inp.T, 16, rng)
        err = _check_rows(wl, r["sout"][ts],
                          lambda q: O.swiglu_expert(inp.xv[ts], *W.get_shared(), act_quant=q), "shared")
        worst = max(worst, err)
    return worst


def boundary_rows(lo, hi):
    """An expert's first and last rows and the rows on each side of the
    kernels' chunk and tile boundaries (16, 32 and 128 rows)."""
    rows = {lo, hi - 1}
    for b in (16, 32, 128):
        rows |= {lo + b - 1, lo + b}
    return sorted(r for r in rows if lo <= r < hi)


def check_ffn_rows(wl, inp: Inputs, r, W: Weights, tok, nthreads=None):
    """Every touched expert on its boundary rows, and the shared expert on its
    first and last tokens, against the C++ oracle reading the weights in their
    storage format (bf16 bits, or E4M3 codes and block scales)."""
    E = wl.num_experts
    off = r["offset"]
    wdt = wl.weight_dtype
    worst, n = 0.0, 0
    if nthreads is None:
        import os
        nthreads = min(16, os.cpu_count() or 1)  # a GPU machine's CPU share

    def ref(rows_x, pair, q):
        a, b = pair
        if wdt == "fp8":
            return R.swiglu_storage(rows_x, a[0], b[0], "fp8", a[1], b[1], act_quant=q, nthreads=nthreads)
        return R.swiglu_storage(rows_x, a, b, wdt, act_quant=q, nthreads=nthreads)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = boundary_rows(lo, hi)
        xs = inp.xv[tok[rows]]
        err = _check_rows(wl, r["eout"][rows], lambda q: ref(xs, W.host[e], q), e)
        worst, n = max(worst, err), n + 1
    if wl.num_shared:
        ts = sorted({0, inp.T - 1})
        err = _check_rows(wl, r["sout"][ts], lambda q: ref(inp.xv[ts], W.host["shared"], q), "shared")
        worst = max(worst, err)
    return worst, n


def check_layer(wl, inp: Inputs, y, idx_gpu, W: Weights, tokens):
    """y on the given tokens against the oracle's dense per-token path under
    the GPU's routing (identical to the oracle's own routing wherever
    check_route found no near-tie)."""
    w_ref = O.gate_weights(inp.logits, idx_gpu, wl)
    yv = y_values(wl, y)
    assert np.isfinite(yv[tokens]).all()

    def ref(q):
        return np.stack([O.dense_token(inp.xv[t], idx_gpu[t], w_ref[t], W.get_expert,
                                       W.get_shared if wl.num_shared else None, act_quant=q) for t in tokens])
    return _check_rows(wl, yv[tokens], ref, "layer", layer=True)


def check_layer_all(wl, inp: Inputs, y, idx_gpu, W: Weights):
    """Every output of y against the oracle's whole layer under the GPU's
    routing (exact activations; E4M3 layers also against the quantised form).
    Returns (error against exact activations, error against the quantised
    form or None)."""
    w_ref = O.gate_weights(inp.logits, idx_gpu, wl)
    yv = y_values(wl, y)
    assert np.isfinite(yv).all()

    def ref(q):
        return O.layer(inp.xv, inp.logits, inp.bias, wl, W.get_expert, W.get_shared if wl.num_shared else None,
                       idx=idx_gpu, w=w_ref, act_quant=q)
    err = _check_rows(wl, yv, ref, "layer", layer=True)
    errq = rel_err(yv, ref(True)) if wl.weight_dtype == "fp8" else None
    return err, errq


def fmt_err(err, errq):
    return f"{err:.2e}" + (f" (quantised form {errq:.2e})" if errq is not None else "")
