"""GPU parity of the masked dispatch layout, through the C ABI.

Masked layout: expert e owns rows [e*T, e*T + count[e]) of an E*T-row
buffer, and a token's row is its expert times T plus its ticket, so the
router writes the token itself (moe_route_dispatch, one launch).  Checked:
routing against the oracle as for the compact layout; every routed row
written exactly once with the token's bytes (E4M3 codes and scales on the
fp8 path), every other row left at its sentinel; expert and layer outputs
against the oracle; and moe_layer in the masked layout bit-identical to
moe_layer in the compact one (each row's arithmetic does not depend on where
the row sits)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_case import (TOL, Inputs, Weights, _check_rows, check_layer, check_layer_all, check_route, cfg_of,
                      fmt_err, host, rel_err, sample, say, y_values)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS
_ES = {"f32": 4, "bf16": 2, "fp8": 1}

CASES = {
    "tiny": WL["tiny"],
    "qwen3": WL["qwen3"],
    "dsv3": WL["dsv3"],
    "dsv3_fp8": WL["dsv3_fp8"],
    "fp8_small": WL["dsv3_fp8"].with_(name="fp8_small", num_experts=32, top_k=4, d_model=512, d_ff=256,
                                      d_ff_shared=512, n_group=4, topk_group=2),
    # E4M3 with many rows per expert (32-row chunks)
    "fp8_rows": WL["dsv3_fp8"].with_(name="fp8_rows", num_experts=16, top_k=4, d_model=768, d_ff=256,
                                     d_ff_shared=512, n_group=4, topk_group=2),
    # bf16, shared expert, d_model >= 1024: the router runs next to the
    # shared expert's gate/up pass
    "cosched": WL["dsv3"].with_(name="cosched", num_experts=16, top_k=4, d_model=1024, d_ff=256,
                                d_ff_shared=512, n_group=4, topk_group=2),
    # many rows per expert: the LDS-tiled GEMMs
    "tiled_small": WL["dsv3"].with_(name="tiled_small", num_experts=8, top_k=2, d_model=256, d_ff=128,
                                    d_ff_shared=256, n_group=2, topk_group=1),
    "softmax_sel": WL["qwen3"].with_(name="softmax_sel", num_experts=64, top_k=6, d_model=384, d_ff=256,
                                     weight="softmax_selected"),
}


def masked_cfg(wl):
    cfg = cfg_of(wl)
    cfg.masked_layout = 1
    return cfg


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


_weights = {}


def weights_for(wl, experts):
    W = _weights.get(wl.name)
    if W is None:
        W = _weights.setdefault(wl.name, Weights(wl, experts=[]))
    W.ensure(experts)
    return W


def run_masked(wl, inp, W=None, fused=True, pad_rows=16):
    import combine_experts_amd as M
    cfg = masked_cfg(wl)
    T, E, k, d = inp.T, wl.num_experts, wl.top_k, wl.d_model
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    tw = torch.full((T, k), float("nan"), device="cuda")
    count = torch.zeros(E, dtype=torch.int32, device="cuda")
    ticket = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    row_of = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    rows = M.moe_dispatch_rows(cfg, T)
    fp8 = wl.weight_dtype == "fp8"
    rdt = "fp8" if fp8 else wl.act_dtype
    recv = torch.full((rows + pad_rows, d * _ES[rdt]), 0x7F, dtype=torch.uint8, device="cuda")
    recv_scale = torch.full((rows + pad_rows, d // 128), float("nan"), device="cuda") if fp8 else None
    if fused:
        M.moe_route_dispatch(cfg, T, inp.logits_d, inp.bias_d, inp.x, idx, tw, count, ticket, recv, recv_scale,
                             row_of)
    else:
        M.moe_route(cfg, T, inp.logits_d, inp.bias_d, idx, tw, count, ticket)
        M.moe_dispatch(cfg, T, inp.x, idx, count, ticket, recv, recv_scale, None, row_of)
    torch.cuda.synchronize()
    r = dict(idx=host(idx), w=host(tw), count=host(count), ticket=host(ticket), row_of=host(row_of),
             recv=host(recv), rows=rows)
    if fp8:
        r["recv_scale"] = host(recv_scale)
    if W is None:
        return r
    eout = torch.full((E * T, d), float("nan"), device="cuda")
    sout = torch.full((T, d), float("nan"), device="cuda") if wl.num_shared else None
    nbytes = M.moe_ffn_workspace_size(cfg, T)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    # masked layout: the GEMMs take the counters where the compact layout
    # passes offsets
    M.moe_expert_ffn(cfg, T, recv, recv_scale, count, W.moe_weights(), inp.x, eout, sout, ws, nbytes)
    ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16
    y = torch.empty((T, d), dtype=ydt, device="cuda")
    M.moe_combine(cfg, T, eout, row_of, tw, sout, y, count)
    torch.cuda.synchronize()
    r.update(eout=host(eout), y=host(y), count_after=host(count))
    if sout is not None:
        r["sout"] = host(sout)
    return r


def check_masked_dispatch(wl, inp, r):
    """Rows e*T + ticket, the oracle's token set per expert, every routed row
    written once with the token's bytes, every other row untouched.  Returns
    the token of each written row (-1 elsewhere)."""
    T, E, k, d = inp.T, wl.num_experts, wl.top_k, wl.d_model
    idx, cnt = r["idx"], r["count"]
    assert np.array_equal(r["row_of"], idx * T + r["ticket"])
    _, offsets, _, tok_ref = O.dispatch(idx, E)
    tok = np.full(E * T, -1, dtype=np.int64)
    tok[r["row_of"].reshape(-1)] = np.repeat(np.arange(T), k)
    assert (tok >= 0).sum() == T * k  # no two slots share a row
    for e in range(E):
        seg = tok[e * T:(e + 1) * T]
        assert (seg[:cnt[e]] >= 0).all() and (seg[cnt[e]:] < 0).all(), e
        assert np.array_equal(np.sort(seg[:cnt[e]]), tok_ref[offsets[e]:offsets[e + 1]]), e
    written = tok >= 0
    recv = r["recv"]
    if wl.weight_dtype == "fp8":
        codes, scales = O.quantize_rows_1x128(inp.xv.astype(np.float32))
        assert np.array_equal(recv[:E * T][written], codes[tok[written]]), "E4M3 codes differ"
        assert np.array_equal(r["recv_scale"][:E * T][written], scales[tok[written]]), "E4M3 scales differ"
        assert (recv[:E * T][~written] == 0x7F).all()
        if wl.num_shared:
            assert np.array_equal(recv[E * T:E * T + T], codes)
            assert np.array_equal(r["recv_scale"][E * T:E * T + T], scales)
        assert (recv[r["rows"]:] == 0x7F).all()
    else:
        xb = np.ascontiguousarray(inp.x_host).view(np.uint8).reshape(T, -1)
        assert np.array_equal(recv[:E * T][written], xb[tok[written]])
        assert (recv[:E * T][~written] == 0x7F).all()
        assert (recv[E * T:] == 0x7F).all()
    return tok


ROUTE_DISPATCH = [("tiny", 16), ("tiny", 129), ("qwen3", 1), ("qwen3", 8), ("qwen3", 128), ("dsv3", 1),
                  ("dsv3", 32), ("dsv3_fp8", 32), ("dsv3_fp8", 512), ("fp8_small", 37), ("softmax_sel", 50),
                  ("cosched", 45)]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("name,T", ROUTE_DISPATCH)
def test_masked_route_dispatch(name, T, fused):
    wl = CASES[name]
    inp = Inputs(wl, T)
    r = run_masked(wl, inp, fused=fused)
    check_route(wl, inp, r)
    check_masked_dispatch(wl, inp, r)


LAYER = [("tiny", 16), ("tiny", 1), ("qwen3", 8), ("qwen3", 3), ("fp8_small", 37), ("fp8_rows", 200),
         ("cosched", 45), ("cosched", 1), ("tiled_small", 300), ("softmax_sel", 50)]


@pytest.mark.parametrize("name,T", LAYER)
def test_masked_chain_against_oracle(name, T):
    wl = CASES[name]
    inp = Inputs(wl, T)
    idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
    W = weights_for(wl, np.unique(idx_ref))
    r = run_masked(wl, inp)
    W.ensure(np.unique(r["idx"]))
    r = run_masked(wl, inp, W)
    check_route(wl, inp, r)
    tok = check_masked_dispatch(wl, inp, r)
    worst = 0.0
    for e in np.unique(r["idx"]):
        rows = np.arange(e * T, e * T + r["count"][e])
        err = _check_rows(wl, r["eout"][rows],
                          lambda q: O.swiglu_expert(inp.xv[tok[rows]], *W.get_expert(int(e)), act_quant=q), e)
        worst = max(worst, err)
    e2, e2q = check_layer_all(wl, inp, r["y"], r["idx"], W)
    assert (r["count_after"] == 0).all()
    say(f"  masked {name} T={T}: ffn err {worst:.2e}, y err {fmt_err(e2, e2q)}")


def _moe_layer(wl, cfg, inp, W, ws):
    import combine_experts_amd as M
    ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16
    y = torch.empty((inp.T, wl.d_model), dtype=ydt, device="cuda")
    M.moe_layer(cfg, inp.T, inp.x, inp.logits_d, inp.bias_d, W.moe_weights(), y, ws, ws.numel())
    torch.cuda.synchronize()
    return host(y)


SAME = [("tiny", (129, 16, 1)), ("qwen3", (128, 8, 1)), ("fp8_small", (37, 5)), ("fp8_rows", (200, 67)),
        ("cosched", (45, 7, 1)), ("tiled_small", (300, 129)), ("dsv3", (128, 1)), ("dsv3_fp8", (32,))]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,Ts", SAME)
def test_masked_layer_equals_compact(name, Ts):
    """One zero-filled workspace per layout serves calls of decreasing size;
    every call gives the same bytes in both layouts."""
    import combine_experts_amd as M
    wl = CASES[name]
    cm, cc = masked_cfg(wl), cfg_of(wl)
    wsm = torch.zeros(M.moe_workspace_size(cm, max(Ts)), dtype=torch.uint8, device="cuda")
    wsc = torch.zeros(M.moe_workspace_size(cc, max(Ts)), dtype=torch.uint8, device="cuda")
    for T in Ts:
        inp = Inputs(wl, T, seed=T)
        idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
        W = weights_for(wl, np.unique(idx_ref))
        r = run_masked(wl, inp)
        W.ensure(np.unique(r["idx"]))
        ym = _moe_layer(wl, cm, inp, W, wsm)
        yc = _moe_layer(wl, cc, inp, W, wsc)
        assert np.isfinite(y_values(wl, ym)).all()
        assert np.array_equal(ym, yc), T
        ym2 = _moe_layer(wl, cm, inp, W, wsm)
        assert np.array_equal(ym2, ym), T
        if T == max(Ts):
            toks = sample(T, 4, np.random.default_rng(T))
            e = check_layer(wl, inp, ym, r["idx"], W, toks)
            say(f"  {name} T={T}: masked == compact, y err (sampled) {e:.2e}")
