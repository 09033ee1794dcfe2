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

# max |err| / max |ref| bounds per weight dtype: bf16 and fp8 as the layer's
# accuracy target states; fp32 from the arithmetic (fp32 accumulation over
# K <= 2048 terms of O(1) products keeps relative errors near 1e-6).
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
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
        # the GPU's choice must still be a valid selection
        for t in np.nonzero(diff)[0]:
            assert len(set(idx[t])) == k and ((idx[t] >= 0) & (idx[t] < E)).all()
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


def check_ffn(wl, inp: Inputs, r, W: Weights, tok, max_experts=None, rng=None):
    """Expert outputs of whole experts (all, or a sample) against the oracle's
    SwiGLU expert on the same rows; shared expert on sampled tokens."""
    rng = rng or np.random.default_rng(0)
    E = wl.num_experts
    q = wl.weight_dtype == "fp8"
    off = r["offset"]
    active = [e for e in range(E) if off[e + 1] > off[e]]
    if max_experts is not None and len(active) > max_experts:
        big = max(active, key=lambda e: off[e + 1] - off[e])
        pick = set(rng.choice(active, size=max_experts - 1, replace=False).tolist()) | {big}
        active = sorted(pick)
    worst = 0.0
    for e in active:
        lo, hi = off[e], off[e + 1]
        ref = O.swiglu_expert(inp.xv[tok[lo:hi]], *W.get_expert(e), act_quant=q)
        err = rel_err(r["eout"][lo:hi], ref)
        worst = max(worst, err)
        assert err <= TOL[wl.weight_dtype], (e, err)
    if wl.num_shared:
        ts = sample(inp.T, 16, rng)
        ref = O.swiglu_expert(inp.xv[ts], *W.get_shared(), act_quant=q)
        err = rel_err(r["sout"][ts], ref)
        worst = max(worst, err)
        assert err <= TOL[wl.weight_dtype], ("shared", err)
    return worst


def check_layer(wl, inp: Inputs, y, idx_gpu, W: Weights, tokens):
    """y on the given tokens against the oracle's dense per-token path under
    the GPU's routing (identical to the oracle's own routing wherever
    check_route found no near-tie)."""
    q = wl.weight_dtype == "fp8"
    w_ref = O.gate_weights(inp.logits, idx_gpu, wl)
    yv = y_values(wl, y)
    ref = np.stack([O.dense_token(inp.xv[t], idx_gpu[t], w_ref[t], W.get_expert,
                                  W.get_shared if wl.num_shared else None, act_quant=q) for t in tokens])
    err = rel_err(yv[tokens], ref)
    assert np.isfinite(yv[tokens]).all()
    assert err <= TOL[wl.weight_dtype], err
    return err
