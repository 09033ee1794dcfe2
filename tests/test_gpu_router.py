"""The router's logits x W_r^T on the GPU, through the C ABI ("7.13 Serving
Mixture-of-Experts", moe_ep_layer listing: the router is a linear map from
the token to one score per expert, then softmax and top-k).

The GPU forms the products (exact for bf16 x bf16) and sums them in fp32, in
an order of its own.  For any order, the error of K products summed with a
rounding at each product and each addition is at most gamma_{K+1} * sum_c
|x_c w_c|, gamma_n = n u / (1 - n u); u = 2^-23 covers both rounding to
nearest and truncation.  Every logit must lie within that bound of the
oracle's float64 product.  Routing from those logits may then differ from routing on
the exact logits only for tokens whose deciding keys (k-th against (k+1)-th
expert, or the group boundary) are closer than the keys can move."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from moe_case import TIE, cfg_of, dev, host, say, x_values
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

WL = mi.WORKLOADS
CASES = {
    "qwen3": WL["qwen3"],
    "dsv3": WL["dsv3"],
    "dsv3_prefill": WL["dsv3_prefill"],
    # the fp32 layer's widths with 64 experts (the router GEMM needs E % 64 == 0)
    "f32_64": WL["tiny"].with_(name="f32_64", num_experts=64, top_k=4, x_std=1.0),
    # bf16, 64 experts: many tokens still take the streaming kernel (the tiled
    # one needs E % 128 == 0)
    "bf16_64": WL["qwen3"].with_(name="bf16_64", num_experts=64, top_k=4),
    # 512 experts: two 256-wide expert tiles per token tile in the tiled and split passes
    "e512": WL["dsv3"].with_(name="e512", num_experts=512, n_group=8, topk_group=4),
}


def fp32_sum_bound(xv, wv):
    n = xv.shape[1] + 1
    u = 2.0 ** -23
    return (n * u / (1.0 - n * u)) * (np.abs(xv) @ np.abs(wv).T)


@pytest.mark.parametrize("name,T", [("qwen3", 1), ("qwen3", 37), ("qwen3", 128), ("qwen3", 512), ("dsv3", 1),
                                    ("dsv3", 8), ("dsv3", 128), ("dsv3_prefill", 4096), ("f32_64", 16),
                                    ("f32_64", 129), ("bf16_64", 300), ("dsv3", 300), ("dsv3", 2048), ("qwen3", 2048),
                                    ("qwen3", 16), ("qwen3", 17), ("dsv3", 16), ("dsv3", 17)])
def test_router_logits(name, T):
    import combine_experts_amd as M
    say(f"\n[gpu-test] router logits {name} T={T}")
    wl = CASES[name]
    x, wr = mi.gen_x(wl, T), mi.gen_router_weight(wl)
    xd, wd = dev(x), dev(wr)
    run = lambda out: M.moe_router_logits(cfg_of(wl), T, xd, wd, out)
    _check_logits(wl, T, x, wr, run)


@pytest.mark.parametrize("name,T", [("dsv3_prefill", 4096), ("dsv3", 2048), ("dsv3", 2176), ("dsv3", 300),
                                    ("dsv3", 256), ("qwen3", 1024), ("qwen3", 2048), ("qwen3", 4100),
                                    ("bf16_64", 2048), ("qwen3", 300), ("dsv3", 255), ("dsv3", 16),
                                    ("e512", 512), ("e512", 2100)])
def test_router_logits_split(name, T):
    """moe_router_logits_ws: the reduction split over workgroups into fp32
    partial sums, added in part order by a second launch (bf16, E % 128 ==
    0, from 256 tokens when d_model >= 4096, else from 1024; elsewhere it is
    moe_router_logits).  The same bound
    against the oracle, reproducible bits, a workspace poisoned with NaN
    first (every partial is written before it is read)."""
    import combine_experts_amd as M
    say(f"\n[gpu-test] split router logits {name} T={T}")
    wl = CASES[name]
    cfg = cfg_of(wl)
    nb = M.moe_router_workspace_size(cfg, T)
    split = wl.num_experts % 128 == 0 and T >= (256 if wl.d_model >= 4096 else 1024)
    assert (nb > 0) == split
    ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    x, wr = mi.gen_x(wl, T), mi.gen_router_weight(wl)
    xd, wd = dev(x), dev(wr)
    run = lambda out: M.moe_router_logits_ws(cfg, T, xd, wd, out, ws if nb else None, nb)
    got = _check_logits(wl, T, x, wr, run)
    if not split:  # the call is moe_router_logits
        plain = torch.empty_like(got)
        M.moe_router_logits(cfg, T, xd, wd, plain)
        torch.cuda.synchronize()
        assert np.array_equal(host(plain).view(np.uint32), host(got).view(np.uint32))


def _check_logits(wl, T, x, wr, run):
    E = wl.num_experts
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    run(out)
    again = torch.full_like(out, float("nan"))
    run(again)
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    assert np.array_equal(host(out).view(np.uint32), host(again).view(np.uint32)), "not reproducible"
    xv, wv = x_values(wl, x), x_values(wl, wr)
    ref = O.router_logits(xv, wv)
    bound = fp32_sum_bound(xv, wv)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err / bound).max())
    # routing from the GPU's logits against routing from the exact ones
    bias = mi.gen_bias(wl)
    idx_gpu, _, _ = O.route(host(out), bias, wl)
    idx_ref, _, info = O.route(ref.astype(np.float32), bias, wl)
    moved = bound.max(axis=1) + np.abs(ref).max(axis=1) * 2.0 ** -24  # fp32 rounding of the logit too
    # keys move at most as much as the logits (the sigmoid's slope is at most
    # 1/4); a group score is a sum of two keys
    slack = 4.0 * moved + TIE
    differ = (np.sort(idx_gpu, axis=1) != np.sort(idx_ref, axis=1)).any(axis=1)
    margin = O.routing_margins(info, wl)
    assert not (differ & ~(margin <= slack)).any()
    say(f"  max |err| / bound = {float((err / bound).max()):.3f}, max |err| = {float(err.max()):.2e}, "
        f"{int(differ.sum())} of {T} tokens route differently (all near ties)")
    return out
