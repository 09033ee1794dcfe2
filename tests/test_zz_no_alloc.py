"""moe_layer_static, the entry point that allocates nothing (its intermediates
live in the library's own scratch array), against moe_layer on a caller
workspace, through the C ABI: bit-identical outputs on consecutive calls of
decreasing size, in both dispatch layouts; calls that need more than the
scratch are refused before anything is launched."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_case import Inputs, Weights, cfg_of, host, say
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS
CASES = {
    "cosched": WL["dsv3"].with_(name="cosched", num_experts=16, top_k=4, d_model=1024, d_ff=256,
                                d_ff_shared=512, n_group=4, topk_group=2),
    "fp8_small": WL["dsv3_fp8"].with_(name="fp8_small", num_experts=32, top_k=4, d_model=512, d_ff=256,
                                      d_ff_shared=512, n_group=4, topk_group=2),
    "tiled_small": WL["dsv3"].with_(name="tiled_small", num_experts=8, top_k=2, d_model=256, d_ff=128,
                                    d_ff_shared=256, n_group=2, topk_group=1),
    "qwen3": WL["qwen3"],
    "tiny": WL["tiny"],
}


def _run(wl, cfg, inp, W, static):
    import combine_experts_amd as M
    ydt = torch.float32 if wl.act_dtype == "f32" else torch.int16
    y = torch.full((inp.T, wl.d_model), -1, dtype=ydt, device="cuda")
    if static:
        M.moe_layer_static(cfg, inp.T, inp.x, inp.logits_d, inp.bias_d, W.moe_weights(), y)
    else:
        nb = M.moe_workspace_size(cfg, inp.T)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        M.moe_layer(cfg, inp.T, inp.x, inp.logits_d, inp.bias_d, W.moe_weights(), y, ws, nb)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("name,Ts,masked", [("cosched", (45, 7), False), ("cosched", (9, 1), True),
                                             ("fp8_small", (37, 5), False), ("tiled_small", (300, 129), False),
                                             ("qwen3", (128, 8), False), ("qwen3", (8, 1), True),
                                             ("tiny", (129, 16), False)])
def test_static_scratch_equals_moe_layer(name, Ts, masked):
    wl = CASES[name]
    cfg = cfg_of(wl)
    cfg.masked_layout = 1 if masked else 0
    W = Weights(wl, experts=[])
    for T in Ts + Ts[:1]:  # the first size again after the smaller one
        say(f"  moe_layer_static {name} T={T} {'masked' if masked else 'compact'}")
        inp = Inputs(wl, T, seed=T)
        idx, _, _ = O.route(inp.logits, inp.bias, wl)
        W.ensure(np.unique(idx))
        y_ref = _run(wl, cfg, inp, W, static=False)
        y = _run(wl, cfg, inp, W, static=True)
        assert np.array_equal(y, y_ref), (name, T)


def test_static_scratch_refuses_oversized_calls():
    import combine_experts_amd as M
    cfg = cfg_of(WL["dsv3"])
    T = 1024
    assert M.moe_workspace_size(cfg, T) > M.moe_layer_static_max_bytes()
    W = M.MoeWeights()
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_static(cfg, T, 0, 0, None, W, 0)
    assert e.value.status == M.MOE_ERR_SCRATCH_LIMIT
