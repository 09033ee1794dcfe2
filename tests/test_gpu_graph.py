"""moe_layer captured in a HIP graph.

moe_layer only enqueues kernels (no allocation, no memset, no host sync)
and leaves its workspace counters at zero, so one capture can be replayed
for new inputs of the same shape.  Each replay runs with new tokens and
logits copied into the captured buffers, with eager work and host
synchronisations between replays, and must give exactly the bytes of an
eager moe_layer call on the same inputs."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_case import Inputs, Weights, cfg_of, host, say
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS
CASES = {
    "qwen3": WL["qwen3"],
    "cosched": WL["dsv3"].with_(name="cosched", num_experts=16, top_k=4, d_model=1024, d_ff=256,
                                d_ff_shared=512, n_group=4, topk_group=2),
    "fp8_small": WL["dsv3_fp8"].with_(name="fp8_small", num_experts=32, top_k=4, d_model=512, d_ff=256,
                                      d_ff_shared=512, n_group=4, topk_group=2),
    "tiled_small": WL["dsv3"].with_(name="tiled_small", num_experts=8, top_k=2, d_model=256, d_ff=128,
                                    d_ff_shared=256, n_group=2, topk_group=1),
}


@pytest.mark.parametrize("masked", [False, True], ids=["compact", "masked"])
@pytest.mark.parametrize("name,T", [("qwen3", 8), ("qwen3", 128), ("cosched", 45), ("fp8_small", 37),
                                    ("tiled_small", 300)])
def test_graph_replays_match_eager(name, T, masked):
    import combine_experts_amd as M
    say(f"\n[gpu-test] graph {name} T={T} masked={masked}")
    wl = CASES[name]
    cfg = cfg_of(wl)
    cfg.masked_layout = 1 if masked else 0
    seeds = (11, 12, 13)
    inps = [Inputs(wl, T, seed=s) for s in seeds]
    experts = set()
    for inp in inps:
        experts |= set(np.unique(O.route(inp.logits, inp.bias, wl)[0]).tolist())
    W = Weights(wl, experts=sorted(experts))
    ws_bytes = M.moe_workspace_size(cfg, T)
    ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16

    def eager(inp):
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        y = torch.empty((T, wl.d_model), dtype=ydt, device="cuda")
        M.moe_layer(cfg, T, inp.x, inp.logits_d, inp.bias_d, W.moe_weights(), y, ws, ws_bytes)
        torch.cuda.synchronize()
        return host(y)

    want = [eager(inp) for inp in inps]
    # captured buffers
    x = inps[0].x.clone()
    logits = inps[0].logits_d.clone()
    bias = inps[0].bias_d.clone() if inps[0].bias_d is not None else None
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, wl.d_model), dtype=ydt, device="cuda")
    weights = W.moe_weights()
    # one eager call on the capture buffers first (the library's per-kernel
    # launch-shape queries run outside the capture)
    M.moe_layer(cfg, T, x, logits, bias, weights, y, ws, ws_bytes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.moe_layer(cfg, T, x, logits, bias, weights, y, ws, ws_bytes)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, inp in enumerate(inps):
            x.copy_(inp.x)
            logits.copy_(inp.logits_d)
            if bias is not None:
                bias.copy_(inp.bias_d)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = host(y)
            assert np.array_equal(got, want[i]), (rep, i)
            # unrelated eager work between replays
            (torch.randn(1 << 16, device="cuda") * 2).sum().item()
    say(f"  {name} T={T}: 6 replays equal the eager calls")


@pytest.mark.parametrize("T", [8, 40])
def test_graph_router_gemm_then_layer(T):
    """moe_router_logits then moe_layer, from hidden states, in one capture:
    every replay equals the eager pair on the same tokens (T = 8 takes the
    dot-product router kernel, T = 40 the streaming one)."""
    import combine_experts_amd as M
    from moe_case import dev
    say(f"\n[gpu-test] graph router GEMM + layer T={T}")
    wl = WL["dsv3"].with_(name="router_graph", num_experts=64, top_k=4, d_model=1024, d_ff=256,
                          d_ff_shared=512, n_group=4, topk_group=2)
    cfg = cfg_of(wl)
    wr = dev(mi.gen_router_weight(wl))
    inps = [Inputs(wl, T, seed=s) for s in (21, 22, 23)]
    ws_bytes = M.moe_workspace_size(cfg, T)
    W = Weights(wl, experts=[])

    def run(x, logits, y, ws):
        M.moe_router_logits(cfg, T, x, wr, logits)
        M.moe_layer(cfg, T, x, logits, inps[0].bias_d, W.moe_weights(), y, ws, ws_bytes)

    # the experts the router picks, so that their weights are in place
    for inp in inps:
        lg = torch.empty((T, wl.num_experts), dtype=torch.float32, device="cuda")
        M.moe_router_logits(cfg, T, inp.x, wr, lg)
        torch.cuda.synchronize()
        W.ensure(np.unique(O.route(host(lg), inps[0].bias, wl)[0]))  # the bias run() passes

    def eager(inp):
        lg = torch.empty((T, wl.num_experts), dtype=torch.float32, device="cuda")
        y = torch.empty((T, wl.d_model), dtype=torch.int16, device="cuda")
        run(inp.x, lg, y, torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        return host(y)

    want = [eager(inp) for inp in inps]
    for w in want:  # every expert the layer used holds real weights
        assert np.isfinite(mi.bf16_bits_to_f32(w)).all()
    x = inps[0].x.clone()
    logits = torch.empty((T, wl.num_experts), dtype=torch.float32, device="cuda")
    y = torch.empty((T, wl.d_model), dtype=torch.int16, device="cuda")
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    run(x, logits, y, ws)  # launch-shape queries outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(x, logits, y, ws)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, inp in enumerate(inps):
            x.copy_(inp.x)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(y), want[i]), (rep, i)
            (torch.randn(1 << 16, device="cuda") * 2).sum().item()
    say(f"  router GEMM + layer T={T}: 6 replays equal the eager calls")


def test_graph_split_router_gemm():
    """moe_router_logits_ws with its reduction split (two launches: partial
    sums, then their sum in part order) captured once: every replay on new
    tokens equals the eager call bit for bit."""
    import combine_experts_amd as M
    from moe_case import dev
    say("\n[gpu-test] graph split router GEMM")
    wl = WL["dsv3"].with_(name="router_split_graph", num_experts=128, top_k=4, d_model=4096, d_ff=256,
                          d_ff_shared=0, num_shared=0, n_group=4, topk_group=2)
    cfg = cfg_of(wl)
    T = 256
    nb = M.moe_router_workspace_size(cfg, T)
    assert nb > 0  # 256 tokens at d_model 4096 take the split
    wr = dev(mi.gen_router_weight(wl))
    xs = [dev(mi.gen_x(wl, T, seed=s)) for s in (31, 32, 33)]
    ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device="cuda")

    def eager(x):
        out = torch.full((T, wl.num_experts), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_router_logits_ws(cfg, T, x, wr, out, ws, nb)
        torch.cuda.synchronize()
        return host(out)

    want = [eager(x) for x in xs]
    x = xs[0].clone()
    out = torch.empty((T, wl.num_experts), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.moe_router_logits_ws(cfg, T, x, wr, out, ws, nb)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(xi)
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(out).view(np.uint32), want[i].view(np.uint32)), (rep, i)
            (torch.randn(1 << 16, device="cuda") * 2).sum().item()
    say("  split router GEMM: 6 replays equal the eager calls")
