"""GPU parity of every entry point against the CPU oracle, through the C ABI.

Routing indices, per-expert counts and the token-ordered dispatch layout are
compared bit-exactly (a routing choice may differ only at an oracle near-tie);
expert outputs and layer outputs within max|err|/max|ref| of 1e-4 (fp32),
2e-2 (bf16) and 6e-2 (fp8).  Experts that no token picks hold NaN weights,
so a kernel that read them would fail every output check."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_case import (TOL, Inputs, Weights, check_dispatch, check_ffn, check_ffn_rows, check_layer,
                      check_layer_all, check_route, cfg_of, fmt_err, host, run_chain, sample, say)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS

# small shapes that exercise odd corners of the configuration space
ODD = {
    "k1_groups": WL["dsv3"].with_(name="k1_groups", num_experts=16, top_k=1, d_model=256, d_ff=128,
                                  d_ff_shared=256, n_group=4, topk_group=2),
    "softmax_sel": WL["qwen3"].with_(name="softmax_sel", num_experts=64, top_k=6, d_model=384, d_ff=256,
                                     weight="softmax_selected"),
    "fp8_small": WL["dsv3_fp8"].with_(name="fp8_small", num_experts=32, top_k=4, d_model=512, d_ff=256,
                                      d_ff_shared=512, n_group=4, topk_group=2),
    "f32_shared": WL["tiny"].with_(name="f32_shared", num_shared=1, d_ff_shared=256, n_group=2, topk_group=1,
                                   bias="normal", bias_std=0.1, routed_scale=2.5, weight="norm_sum"),
    # many rows per expert: takes the LDS-tiled prefill kernel (token tiles of
    # 128 with a ragged last tile, several feature tiles, shared expert)
    "tiled_small": WL["dsv3"].with_(name="tiled_small", num_experts=8, top_k=2, d_model=256, d_ff=128,
                                    d_ff_shared=256, n_group=2, topk_group=1),
    # E4M3 with many rows per expert: the gate/up pass takes 32-row chunks
    "fp8_rows": WL["dsv3_fp8"].with_(name="fp8_rows", num_experts=16, top_k=4, d_model=768, d_ff=256,
                                     d_ff_shared=512, n_group=4, topk_group=2),
    # bf16 with a shared expert and d_model >= 1024: moe_layer runs the shared
    # expert's gate/up pass inside the router's launch
    "cosched": WL["dsv3"].with_(name="cosched", num_experts=16, top_k=4, d_model=1024, d_ff=256,
                                d_ff_shared=512, n_group=4, topk_group=2),
    # d_model not a multiple of 256: the down pass takes 128-row weight tiles
    "tiled_narrow": WL["dsv3"].with_(name="tiled_narrow", num_experts=8, top_k=2, d_model=384, d_ff=256,
                                     d_ff_shared=384, n_group=2, topk_group=1),
    # bf16 activation tiles shared through LDS or not: the gate/up pass has 17
    # K-steps per item, which a 2-way K-split cannot divide (private tiles);
    # the down pass has 16 (shared tiles)
    "share_odd": WL["dsv3"].with_(name="share_odd", num_experts=8, top_k=2, d_model=2176, d_ff=2048,
                                  d_ff_shared=2048, n_group=2, topk_group=1),
    # E4M3 down pass with 9 K-steps: private tiles under a 2-way K-split (few
    # rows per expert), shared by (4, 1) column waves with two or more rows
    # per expert
    "fp8_odd": WL["dsv3_fp8"].with_(name="fp8_odd", num_experts=16, top_k=4, d_model=512, d_ff=2304,
                                    d_ff_shared=2304, n_group=4, topk_group=2),
}


def wl_of(name):
    return WL[name] if name in WL else ODD[name]


ROUTE_CASES = [("tiny", 16), ("tiny", 1), ("tiny", 129), ("qwen3", 1), ("qwen3", 8), ("qwen3", 32),
               ("qwen3", 128), ("qwen3", 3), ("dsv3", 1), ("dsv3", 8), ("dsv3", 32), ("dsv3", 128),
               ("dsv3", 17), ("dsv3_fp8", 512), ("dsv3_prefill", 4096), ("k1_groups", 33),
               ("softmax_sel", 50), ("qwen3", 255), ("qwen3", 256), ("dsv3", 256), ("dsv3", 300)]


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route(name, T):
    wl = wl_of(name)
    inp = Inputs(wl, T)
    r = run_chain(wl, inp, None, stages=("route",))
    diff = check_route(wl, inp, r)
    say(f"  route {name} T={T}: near-tie differences {int(diff.sum())}")


def _adversarial_logits(rng, T, E):
    lg = rng.choice(np.array([-2.0, -0.5, 0.0, 0.25, 1.0], np.float32), size=(T, E))
    lg[0, :] = 0.0                      # all equal
    lg[1, rng.integers(E)] = np.nan
    lg[2, rng.integers(E)] = np.inf
    lg[3, rng.integers(E)] = -np.inf
    lg[4, :] = np.nan                   # all NaN: the lowest eligible indices win
    return lg


@pytest.mark.parametrize("name", ["dsv3", "qwen3", "k1_groups", "tiny"])
def test_route_ties_nan_inf(name):
    """Exact ties, NaN and infinite logits: selection must follow the stated
    tie-break (lower index) and stay in range, bit-exactly like the oracle."""
    wl = wl_of(name)
    T = 64
    rng = np.random.default_rng(5)
    inp = Inputs(wl, T)
    inp.logits = _adversarial_logits(rng, T, wl.num_experts)
    if inp.bias is not None:
        inp.bias = rng.choice(np.array([0.0, 0.125], np.float32), size=wl.num_experts)
        inp.bias_d = torch.from_numpy(inp.bias).cuda()
    inp.logits_d = torch.from_numpy(inp.logits).cuda()
    r = run_chain(wl, inp, None, stages=("route",))
    idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
    assert np.array_equal(r["idx"], idx_ref)
    assert np.array_equal(r["count"], np.bincount(idx_ref.reshape(-1), minlength=wl.num_experts))


DISPATCH_CASES = [("tiny", 16), ("tiny", 129), ("qwen3", 1), ("qwen3", 128), ("dsv3", 8), ("dsv3", 128),
                  ("dsv3_fp8", 32), ("dsv3_fp8", 512), ("dsv3_prefill", 4096), ("fp8_small", 37),
                  ("k1_groups", 33)]


@pytest.mark.parametrize("name,T", DISPATCH_CASES)
def test_dispatch(name, T):
    wl = wl_of(name)
    inp = Inputs(wl, T)
    r = run_chain(wl, inp, None, stages=("route", "dispatch"))
    check_route(wl, inp, r)
    check_dispatch(wl, inp, r)


# ---------------------------------------------------------------------------
# Whole chain and moe_layer on shapes whose oracle runs in seconds
# ---------------------------------------------------------------------------

_weights = {}


def weights_for(wl, experts):
    key = wl.name if wl.name not in ("dsv3_prefill",) else "dsv3"
    W = _weights.get(key)
    if W is None:
        W = Weights(wl, experts=[])
        _weights[key] = W
    W.ensure(experts)
    return W


def _touched(wl, inp):
    idx_ref, _, _ = O.route(inp.logits, inp.bias, wl)
    return set(np.unique(idx_ref).tolist())


SMALL_LAYER = [("tiny", 16), ("tiny", 1), ("tiny", 17), ("tiny", 129), ("qwen3", 1), ("qwen3", 8),
               ("qwen3", 32), ("qwen3", 128), ("qwen3", 3), ("k1_groups", 33), ("softmax_sel", 50),
               ("fp8_small", 1), ("fp8_small", 37), ("f32_shared", 40), ("tiled_small", 300),
               ("tiled_small", 129), ("tiled_small", 1100), ("tiled_narrow", 257), ("qwen3", 512),
               ("fp8_rows", 200), ("fp8_rows", 67), ("cosched", 1), ("cosched", 45), ("cosched", 60),
               ("qwen3", 256),
               ("share_odd", 40), ("fp8_odd", 3), ("fp8_odd", 40),
               # either side of the E4M3 wide-chunk rule (T k >= E: 64-row chunks): 32 experts x 4
               ("fp8_small", 8), ("fp8_small", 7)]


@pytest.mark.parametrize("name,T", SMALL_LAYER)
def test_layer_full_oracle(name, T):
    wl = wl_of(name)
    inp = Inputs(wl, T)
    W = weights_for(wl, _touched(wl, inp))
    r = run_chain(wl, inp, W, stages=("route",))
    W.ensure(np.unique(r["idx"]))
    r = run_chain(wl, inp, W)
    check_route(wl, inp, r)
    tok = check_dispatch(wl, inp, r)
    e1 = check_ffn(wl, inp, r, W, tok)
    e2, e2q = check_layer_all(wl, inp, r["y"], r["idx"], W)
    assert (r["count_after"] == 0).all()
    say(f"  layer {name} T={T}: ffn err {e1:.2e}, y err {fmt_err(e2, e2q)}")


def _layer_via_moe_layer(wl, inp, W, ws=None):
    import combine_experts_amd as M
    cfg = cfg_of(wl)
    nbytes = M.moe_workspace_size(cfg, inp.T)
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16
    y = torch.empty((inp.T, wl.d_model), dtype=ydt, device="cuda")
    M.moe_layer(cfg, inp.T, inp.x, inp.logits_d, inp.bias_d, W.moe_weights(), y, ws, ws.numel())
    torch.cuda.synchronize()
    return host(y), ws


@pytest.mark.parametrize("name,Ts", [("tiny", (129, 16, 1)), ("qwen3", (128, 8, 1)), ("fp8_small", (37, 5)),
                                     ("k1_groups", (33, 2)), ("cosched", (45, 7, 1))])
def test_moe_layer_equals_chain_and_reuses_workspace(name, Ts):
    """moe_layer is bit-identical to the four entry points run in turn (the
    results do not depend on slot order or timing), and one zero-filled
    workspace serves successive calls of decreasing size."""
    wl = wl_of(name)
    ws = None
    import combine_experts_amd as M
    ws = torch.zeros(M.moe_workspace_size(cfg_of(wl), max(Ts)), dtype=torch.uint8, device="cuda")
    for T in Ts:
        inp = Inputs(wl, T, seed=T)
        W = weights_for(wl, _touched(wl, inp))
        r = run_chain(wl, inp, W, stages=("route",))
        W.ensure(np.unique(r["idx"]))
        chain = run_chain(wl, inp, W)
        y, ws = _layer_via_moe_layer(wl, inp, W, ws)
        assert np.array_equal(y, chain["y"]), T
        y2, ws = _layer_via_moe_layer(wl, inp, W, ws)
        assert np.array_equal(y2, y), T


# ---------------------------------------------------------------------------
# Full-size workloads: everything at full size, outputs on sampled tokens
# ---------------------------------------------------------------------------

# dsv3 at 192 tokens: 6 rows per expert, which takes the LDS-tiled kernel at this d_model
BIG_LAYER = [("dsv3", 1), ("dsv3", 8), ("dsv3", 32), ("dsv3", 128), ("dsv3", 192), ("dsv3_fp8", 32),
             ("dsv3_fp8", 128), ("dsv3_fp8", 512), ("dsv3_prefill", 4096)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T", BIG_LAYER)
def test_layer_full_size_sampled(name, T):
    """Full-size layers: routing and dispatch whole; every touched expert on
    its first and last rows and on both sides of the 16-, 32- and 128-row
    chunk and tile boundaries (C++ oracle on the stored weights); the shared
    expert on the first and last tokens; whole experts for a sample (numpy
    oracle); y on sampled tokens through the dense per-token path."""
    wl = wl_of(name)
    inp = Inputs(wl, T)
    say(f"  generating weights for {name} T={T}")
    W = weights_for(wl, _touched(wl, inp))
    r = run_chain(wl, inp, W, stages=("route",))
    W.ensure(np.unique(r["idx"]))
    say(f"  running chain {name} T={T}")
    r = run_chain(wl, inp, W)
    check_route(wl, inp, r)
    tok = check_dispatch(wl, inp, r)
    rng = np.random.default_rng(T)
    e0, n = check_ffn_rows(wl, inp, r, W, tok)
    say(f"  {n} touched experts checked on their boundary rows: worst err {e0:.2e}")
    e1 = check_ffn(wl, inp, r, W, tok, max_experts=4, rng=rng)
    toks = sample(T, 8, rng)
    e2 = check_layer(wl, inp, r["y"], r["idx"], W, toks)
    y, _ = _layer_via_moe_layer(wl, inp, W)
    assert np.array_equal(y, r["y"])
    say(f"  layer {name} T={T}: ffn err {e1:.2e}, y err (sampled) {e2:.2e}")
