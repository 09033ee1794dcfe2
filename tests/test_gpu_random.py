"""Seeded random sweep of the configuration space on the GPU, through the C
ABI, against the oracle: expert counts (E = 8 .. 1024, including counts that
are not multiples of 64), group-limited routing with every group count that
divides E, k from 1 to 16, both score and both weight rules, with and
without bias and shared expert, all three precisions, small and odd model
widths, and token counts from 1 to 257 (which also reach the LDS-tiled
kernel).  Each case checks routing, dispatch layout, expert outputs and the
layer output to the same bar as the named configurations."""
import numpy as np
import pytest

import moe_inputs as mi
from moe_case import (TOL, Inputs, Weights, check_dispatch, check_ffn, check_layer_all, check_route, fmt_err,
                      rel_err, run_chain, say, y_values)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

N_CASES = 24


def random_workload(i):
    rng = np.random.default_rng(1000 + i)
    wdt = str(rng.choice(["f32", "bf16", "bf16", "fp8"]))
    act = "f32" if wdt == "f32" else "bf16"
    mult = {"f32": 64, "bf16": 128, "fp8": 256}[wdt]
    E = int(rng.choice([8, 16, 24, 40, 64, 96, 128, 200, 256, 1024]))
    G = int(rng.choice([g for g in range(1, 65) if E % g == 0]))
    kg = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(16, kg * (E // G)) + 1))
    d = mult * int(rng.integers(1, 4))
    F = mult * int(rng.integers(1, 3))
    shared = int(rng.integers(0, 2))
    Fs = mult * int(rng.integers(1, 3)) if shared else 0
    score = str(rng.choice(["sigmoid", "softmax"]))
    weight = str(rng.choice(["norm_sum", "softmax_selected"]))
    bias = str(rng.choice(["none", "normal"])) if score == "sigmoid" else "none"
    scale = float(rng.choice([1.0, 2.5]))
    T = int(rng.choice([1, 5, 33, 100, 257]))
    wl = mi.Workload(f"rand{i}", E, k, d, F, shared, Fs, G, kg, score, weight, scale, act, wdt,
                     1.0, 0.02, bias, bias_std=0.1)
    return wl, T


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config(i):
    wl, T = random_workload(i)
    say(f"\n[gpu-test] random case {i}: E={wl.num_experts} k={wl.top_k} G={wl.n_group}/{wl.topk_group} "
        f"d={wl.d_model} F={wl.d_ff} shared={wl.num_shared}x{wl.d_ff_shared} {wl.score}/{wl.weight} "
        f"bias={wl.bias} {wl.act_dtype}/{wl.weight_dtype} T={T}")
    inp = Inputs(wl, T, seed=i)
    W = Weights(wl, experts=[])
    r = run_chain(wl, inp, W, stages=("route",))
    W.ensure(np.unique(r["idx"]))
    r = run_chain(wl, inp, W)
    check_route(wl, inp, r)
    tok = check_dispatch(wl, inp, r)
    e1 = check_ffn(wl, inp, r, W, tok)
    e2, e2q = check_layer_all(wl, inp, r["y"], r["idx"], W)
    assert (r["count_after"] == 0).all()
    say(f"  ffn err {e1:.2e}, y err {fmt_err(e2, e2q)}")


# the validated maxima: E = 1024 experts, k = 64 slots (the whole wave picks),
# 64 groups
EDGE = [
    mi.Workload("edge_e1024_k64", 1024, 64, 128, 128, 1, 128, 1, 1, "sigmoid", "norm_sum", 2.5, "bf16", "bf16",
                1.0, 0.02, "normal", bias_std=0.1),
    mi.Workload("edge_g64_k64", 1024, 64, 128, 128, 0, 0, 64, 4, "softmax", "norm_sum", 1.0, "bf16", "bf16",
                1.0, 0.02, "none"),
    mi.Workload("edge_k64_fp8", 128, 64, 256, 256, 1, 256, 8, 8, "sigmoid", "softmax_selected", 1.0, "bf16", "fp8",
                1.0, 0.02, "normal", bias_std=0.1),
]


@pytest.mark.parametrize("wl", EDGE, ids=lambda w: w.name)
@pytest.mark.parametrize("T", [1, 37])
def test_edge_maxima(wl, T):
    say(f"\n[gpu-test] edge {wl.name} T={T}")
    inp = Inputs(wl, T, seed=T)
    W = Weights(wl, experts=[])
    r = run_chain(wl, inp, W, stages=("route",))
    W.ensure(np.unique(r["idx"]))
    r = run_chain(wl, inp, W)
    check_route(wl, inp, r)
    tok = check_dispatch(wl, inp, r)
    check_ffn(wl, inp, r, W, tok)
    e2, e2q = check_layer_all(wl, inp, r["y"], r["idx"], W)
    assert (r["count_after"] == 0).all()
    say(f"  y err {fmt_err(e2, e2q)}")
