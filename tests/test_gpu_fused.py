"""GPU parity of moe_layer_fused (the whole layer in one persistent launch)
through the C ABI.

Checked: the layer's outputs against the oracle under the routing moe_route
picks on the same logits (the fused launch routes with the same selection
code; moe_route's indices are themselves checked against the oracle);
identical bits run to run; identical bits with a workspace whose data regions
(past the sync words) are poisoned with NaN, and after a call on other inputs (no stale reads);
the launch's own router GEMM (from the hidden states) identical to
moe_router_logits followed by the fused layer on its logits; a HIP graph of
the call replayed on new inputs; the sync words (counters, flags, error word)
back at zero after every call.  Experts no token picks hold NaN weights."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_case import Inputs, Weights, cfg_of, check_layer_all, check_route, dev, fmt_err, host, run_chain, say
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS
CASES = {
    "qwen3": WL["qwen3"],
    "dsv3": WL["dsv3"],
    # small shapes: gate/up and down passes with (4, 1) column waves, a shared expert
    "cosched": WL["dsv3"].with_(name="cosched", num_experts=16, top_k=4, d_model=1024, d_ff=256,
                                d_ff_shared=512, n_group=4, topk_group=2),
    # 16 K-steps in the gate/up pass: (2, 2) with shared activation tiles
    "mid": WL["qwen3"].with_(name="mid", num_experts=64, top_k=6, d_model=2048, d_ff=768),
    "softmax_sel": WL["qwen3"].with_(name="softmax_sel", num_experts=64, top_k=6, d_model=384, d_ff=256,
                                     weight="softmax_selected"),
}

_weights = {}


def weights_for(wl, experts):
    W = _weights.get(wl.name)
    if W is None:
        W = _weights.setdefault(wl.name, Weights(wl, experts=[]))
    W.ensure(experts)
    return W


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


def _fused(wl, cfg, inp, W, ws, logits=True, w_router=None):
    import combine_experts_amd as M
    y = torch.full((inp.T, wl.d_model), -1, dtype=torch.int16, device="cuda")
    M.moe_layer_fused(cfg, inp.T, inp.x, inp.logits_d if logits else None, w_router, inp.bias_d, W.moe_weights(), y,
                      ws, ws.numel())
    torch.cuda.synchronize()
    return host(y)


# the workspace's leading words that are zero between calls: an exit count,
# the error word (byte 16) and two 4 KB grid-barrier blocks
SYNC_BYTES = 3 * 4096


def _sync_words(ws):
    return host(ws[:SYNC_BYTES].view(torch.int32))


def _new_ws(cfg, T):
    import combine_experts_amd as M
    return torch.zeros(M.moe_fused_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("name,T", [("qwen3", 1), ("qwen3", 3), ("qwen3", 8), ("qwen3", 16), ("dsv3", 1),
                                    ("dsv3", 8), ("cosched", 1), ("cosched", 13), ("mid", 5),
                                    ("softmax_sel", 16)])
def test_fused_layer_against_oracle(name, T):
    import combine_experts_amd as M
    wl = CASES[name]
    cfg = cfg_of(wl)
    assert M.moe_fused_supported(cfg, T)
    inp = Inputs(wl, T, seed=100 + T)
    idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
    W = weights_for(wl, np.unique(idx_ref))
    r = run_chain(wl, inp, W, stages=("route",))
    check_route(wl, inp, r)
    W.ensure(np.unique(r["idx"]))
    ws = _new_ws(cfg, T)
    say(f"  fused {name} T={T}")
    y = _fused(wl, cfg, inp, W, ws)
    assert not _sync_words(ws).any(), np.nonzero(_sync_words(ws))
    e, eq = check_layer_all(wl, inp, y, r["idx"], W)
    y2 = _fused(wl, cfg, inp, W, ws)
    assert np.array_equal(y2, y)
    # poisoned data regions: every value the launch reads it wrote first
    ws[SYNC_BYTES:].fill_(0xFF)
    torch.cuda.synchronize()
    y3 = _fused(wl, cfg, inp, W, ws)
    assert np.array_equal(y3, y)
    assert not _sync_words(ws).any()
    say(f"  fused {name} T={T}: y err {fmt_err(e, eq)}")


@pytest.mark.parametrize("name,Ts", [("qwen3", (8, 1, 16)), ("cosched", (13, 2))])
def test_fused_layer_consecutive_calls(name, Ts):
    """One workspace across calls of different sizes and inputs: each call
    equals a call on a fresh workspace."""
    wl = CASES[name]
    cfg = cfg_of(wl)
    ws = _new_ws(cfg, max(Ts))
    for T in Ts:
        inp = Inputs(wl, T, seed=7 * T)
        idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
        W = weights_for(wl, np.unique(idx_ref))
        say(f"  fused {name} T={T} reused workspace")
        y = _fused(wl, cfg, inp, W, ws)
        y_fresh = _fused(wl, cfg, inp, W, _new_ws(cfg, T))
        assert np.array_equal(y, y_fresh), T


@pytest.mark.parametrize("name,T", [("qwen3", 1), ("qwen3", 8), ("dsv3", 4), ("mid", 9)])
def test_fused_router_from_hidden_states(name, T):
    """With the router weight in place of the logits, the launch computes the
    logits itself: bit-identical to moe_router_logits followed by the fused
    layer on those logits."""
    import combine_experts_amd as M
    wl = CASES[name]
    cfg = cfg_of(wl)
    inp = Inputs(wl, T, seed=31 + T)
    wr = dev(mi.gen_router_weight(wl))
    logits = torch.empty((T, wl.num_experts), dtype=torch.float32, device="cuda")
    M.moe_router_logits(cfg, T, inp.x, wr, logits)
    torch.cuda.synchronize()
    inp.logits = host(logits)
    inp.logits_d = logits
    idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
    W = weights_for(wl, np.unique(idx_ref))
    r = run_chain(wl, inp, W, stages=("route",))
    W.ensure(np.unique(r["idx"]))
    ws = _new_ws(cfg, T)
    say(f"  fused router {name} T={T}")
    y_router = _fused(wl, cfg, inp, W, ws, logits=False, w_router=wr)
    y_logits = _fused(wl, cfg, inp, W, _new_ws(cfg, T))
    assert np.array_equal(y_router, y_logits)
    assert not _sync_words(ws).any()
    check_layer_all(wl, inp, y_router, r["idx"], W)


def test_fused_layer_graph_replay():
    """The fused call captured once and replayed on new inputs (copied into the
    captured buffers between replays, with eager work in between): every
    replay equals the eager call on the same inputs."""
    import combine_experts_amd as M
    wl = CASES["qwen3"]
    cfg = cfg_of(wl)
    T = 4
    inps = [Inputs(wl, T, seed=s) for s in (1, 2, 3)]
    for inp in inps:
        idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
        W = weights_for(wl, np.unique(idx_ref))
    x = inps[0].x.clone()
    lg = inps[0].logits_d.clone()
    y = torch.empty((T, wl.d_model), dtype=torch.int16, device="cuda")
    ws = _new_ws(cfg, T)
    eager = []
    for inp in inps:
        eager.append(_fused(wl, cfg, inp, W, _new_ws(cfg, T)))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.moe_layer_fused(cfg, T, x, lg, None, None, W.moe_weights(), y, ws, ws.numel(), stream=s)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, inp in enumerate(inps):
            x.copy_(inp.x)
            lg.copy_(inp.logits_d)
            torch.cuda.synchronize()
            say(f"  graph replay {rep}, input {i}")
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(y), eager[i]), (rep, i)
            _ = (x.float().sum()).item()  # eager work between replays
    assert not _sync_words(ws).any()
