"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print, a closed form, a brute-force enumeration on tiny inputs, an
independent formulation, or a property that any correct implementation has.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import moe_inputs as mi
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


class Spec:
    def __init__(self, E, k, G=1, kg=1, score="sigmoid", weight="norm_sum", scale=1.0, shared=0):
        self.num_experts, self.top_k, self.n_group, self.topk_group = E, k, G, kg
        self.score, self.weight, self.routed_scale, self.num_shared = score, weight, scale, shared


# ---------------------------------------------------------------------------
# Expected distinct experts (page 2, "Why MoE Serving Is a Different Problem")
# ---------------------------------------------------------------------------


def test_expected_distinct_printed_instance():
    g = _golden("expected_distinct.json")
    E, k, B = g["E"], g["k"], g["B"]
    assert abs((1 - k / E) ** B - g["printed_miss_probability"]) < 0.001
    v = O.expected_distinct(E, k, B)
    assert abs(v - g["printed_distinct"]) < 0.5
    assert abs(v / E - g["printed_fraction"]) < 0.005


@pytest.mark.parametrize("G,kg", [(1, 1), (8, 4)])
def test_expected_distinct_monte_carlo(G, kg):
    """With zero bias and iid logits every expert is picked with probability
    k/E, also under group-limited routing (symmetry over experts and groups),
    so the mean number of distinct experts per batch of B tokens must match
    E(1 - (1 - k/E)^B) = 222.44 at (256, 8, 64).  2000 batches; the per-batch
    standard deviation is about 4.5, so the mean is good to about 0.1."""
    E, k, B, nb = 256, 8, 64, 2000
    spec = Spec(E, k, G, kg, score="sigmoid")
    logits = mi.normal_f32(11, 2, (nb * B, E), 1.0)
    idx, _, _ = O.route(logits, np.zeros(E, np.float32), spec)
    idx = idx.reshape(nb, B * k)
    distinct = np.array([len(np.unique(r)) for r in idx])
    assert abs(distinct.mean() - O.expected_distinct(E, k, B)) < 0.5


# ---------------------------------------------------------------------------
# Routing against brute force
# ---------------------------------------------------------------------------


def _lex_best(cands, score_of):
    """Brute force: the candidate subset whose members, sorted by (score desc,
    index asc), give the lexicographically largest sequence."""
    def seq(S):
        return sorted(((-score_of[i], i) for i in S))
    best = None
    for S in cands:
        s = seq(S)
        if best is None or s < best[0]:
            best = (s, S)
    return [i for _, i in best[0]]


def _bruteforce_route(keys, E, k, G, kg):
    gsize = E // G
    if G > 1:
        gscore = []
        for q in range(G):
            mem = list(range(q * gsize, (q + 1) * gsize))
            if gsize == 1:
                gscore.append(keys[mem[0]])
            else:
                gscore.append(max(np.float32(keys[a]) + np.float32(keys[b])
                                  for a, b in itertools.combinations(mem, 2)))
        groups = _lex_best(itertools.combinations(range(G), kg), gscore)
        elig = [e for e in range(E) if e // gsize in groups]
    else:
        elig = list(range(E))
    return _lex_best(itertools.combinations(elig, k), keys)


@pytest.mark.parametrize("case", range(60))
def test_route_matches_bruteforce(case):
    rng = np.random.default_rng(1000 + case)
    E = int(rng.choice([4, 8, 12, 16]))
    G = int(rng.choice([g for g in (1, 2, 4) if E % g == 0]))
    kg = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, kg * (E // G) + 1))
    k = min(k, 6)
    T = 5
    # few distinct values: many exact ties; sometimes NaN / +-inf
    logits = rng.choice(np.array([-1.0, -0.25, 0.0, 0.5, 2.0], np.float32), size=(T, E))
    if case % 5 == 0:
        logits[0, rng.integers(E)] = np.nan
        logits[1, rng.integers(E)] = np.inf
        logits[2, rng.integers(E)] = -np.inf
    bias = rng.choice(np.array([0.0, 0.0, 0.125, -0.125], np.float32), size=E)
    score = "softmax" if case % 3 == 0 else "sigmoid"
    spec = Spec(E, k, G, kg, score=score)
    idx, w, info = O.route(logits, bias if score == "sigmoid" else None, spec)
    keys = info["keys"]
    for t in range(T):
        bf = _bruteforce_route([np.float32(v) for v in keys[t]], E, k, G, kg)
        assert list(idx[t]) == bf, (t, keys[t], idx[t], bf)


def test_selection_keys_precision_and_nan():
    spec = Spec(4, 2)
    logits = np.array([[np.nan, 0.0, 1.0, -1.0]], np.float32)
    bias = np.array([0.0, 0.5, 0.0, 0.0], np.float32)
    keys = O.selection_keys(logits, bias, "sigmoid")
    assert keys.dtype == np.float32
    assert keys[0, 0] == -np.inf
    assert keys[0, 1] == np.float32(0.5) + np.float32(0.5)
    assert keys[0, 2] == np.float32(1.0 / (1.0 + math.exp(-1.0)))
    idx, _, _ = O.route(logits, bias, spec)
    assert list(idx[0]) == [1, 2]


def test_softmax_selection_equals_selection_on_probabilities():
    """The moe_ep_layer listing selects on softmax probabilities; the oracle
    selects on logits.  Same order because softmax is strictly increasing."""
    spec = Spec(128, 8, score="softmax")
    logits = mi.gen_logits(mi.WORKLOADS["qwen3"], 512, seed=3)
    idx, _, _ = O.route(logits, None, spec)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    ref = np.argsort(-p, axis=1, kind="stable")[:, :8]
    assert np.array_equal(idx, ref)


def test_softmax_weights_are_softmax_over_selected_logits():
    spec = Spec(128, 8, score="softmax")
    logits = mi.gen_logits(mi.WORKLOADS["qwen3"], 64, seed=4)
    idx, w, _ = O.route(logits, None, spec)
    sel = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-12, atol=1e-15)


def test_softmax_selected_weights_tiny_workload():
    """Tiny workload: softmax over the two selected sigmoid scores."""
    wl = mi.WORKLOADS["tiny"]
    logits = mi.gen_logits(wl, 16)
    idx, w, _ = O.route(logits, mi.gen_bias(wl), wl)
    s = O.sigmoid(np.take_along_axis(logits.astype(np.float64), idx, axis=1))
    ref = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-14)


@pytest.mark.parametrize("name", ["dsv3", "qwen3", "tiny", "dsv3_prefill"])
def test_route_invariants(name):
    wl = mi.WORKLOADS[name]
    T = 256
    logits = mi.gen_logits(wl, T, seed=5)
    idx, w, info = O.route(logits, mi.gen_bias(wl, seed=5), wl)
    E, k = wl.num_experts, wl.top_k
    assert idx.shape == (T, k)
    assert ((idx >= 0) & (idx < E)).all()
    assert all(len(set(r)) == k for r in idx)
    groups = idx // (E // wl.n_group)
    assert all(len(set(r)) <= wl.topk_group for r in groups)
    assert (w >= 0).all()
    assert np.allclose(w.sum(axis=1), wl.routed_scale, rtol=1e-12)
    keys = info["keys"]
    kk = np.take_along_axis(keys, idx, axis=1)
    assert (np.diff(kk, axis=1) <= 0).all()  # ordered by key


# ---------------------------------------------------------------------------
# Dispatch / combine: exact inverse permutation
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (17, 8, 2), (64, 16, 4), (3, 256, 8), (0, 8, 2)])
def test_dispatch_combine_inverse_permutation(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32).reshape(T, k)
    x = rng.standard_normal((T, 24)).astype(np.float32)
    counts, offsets, row_of, tok = O.dispatch(idx, E)
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=E))
    assert counts.sum() == T * k and offsets[-1] == T * k
    # every row written exactly once
    assert sorted(row_of.reshape(-1).tolist()) == list(range(T * k))
    # rows of one expert are contiguous, ascending in token
    for e in range(E):
        toks = tok[offsets[e]:offsets[e + 1]]
        assert list(toks) == sorted(toks)
        assert all(e in idx[t] for t in toks)
    recv = O.gather_rows(x.astype(np.float64), tok)
    for j0 in range(k):
        w = np.zeros((T, k))
        w[:, j0] = 1.0
        y = O.combine(recv, row_of, w)
        assert np.array_equal(y, x.astype(np.float64))


# ---------------------------------------------------------------------------
# Expert FFN
# ---------------------------------------------------------------------------


def _small_layer(seed, E=8, k=2, d=32, F=16, Fs=24, T=19, G=1, kg=1, shared=1):
    rng = np.random.default_rng(seed)
    spec = Spec(E, k, G, kg, scale=2.5, shared=shared)
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    W13 = 0.2 * rng.standard_normal((E, 2 * F, d))
    W2 = 0.2 * rng.standard_normal((E, d, F))
    WS13 = 0.2 * rng.standard_normal((2 * Fs, d))
    WS2 = 0.2 * rng.standard_normal((d, Fs))
    return spec, x, logits, bias, (lambda e: (W13[e], W2[e])), (lambda: (WS13, WS2))


@pytest.mark.parametrize("seed", range(4))
def test_ffn_dispatch_path_equals_dense_per_token(seed):
    spec, x, logits, bias, ge, gs = _small_layer(seed, G=4 if seed % 2 else 1, kg=2 if seed % 2 else 1)
    y = O.layer(x, logits, bias, spec, ge, gs)
    idx, w, _ = O.route(logits, bias, spec)
    for t in range(x.shape[0]):
        yt = O.dense_token(x[t], idx[t], w[t], ge, gs)
        assert np.allclose(y[t], yt, rtol=1e-12, atol=1e-12)


def test_ffn_zero_input_gives_zero():
    spec, x, logits, bias, ge, gs = _small_layer(7)
    y = O.layer(np.zeros_like(x), logits, bias, spec, ge, gs)
    assert np.array_equal(y, np.zeros_like(y))


def test_ffn_zero_up_projection_leaves_shared_only():
    spec, x, logits, bias, ge, gs = _small_layer(8)
    F = 16

    def ge0(e):
        w13, w2 = ge(e)
        w13 = w13.copy()
        w13[F:] = 0.0
        return w13, w2
    y = O.layer(x, logits, bias, spec, ge0, gs)
    ws13, ws2 = gs()
    Fs = ws13.shape[0] // 2
    g = x @ ws13[:Fs].T
    shared = (g / (1 + np.exp(-g)) * (x @ ws13[Fs:].T)) @ ws2.T
    assert np.allclose(y, shared, rtol=1e-13, atol=1e-13)


def test_ffn_scalar_case_by_hand():
    """d = F = 1, one expert, k = 1: y = w * wd * silu(wg * x) * (wu * x).
    x = 1, wg = 1, wu = 2, wd = 3, w = 1: silu(1) = 0.7310585786300049 (the
    logistic function at 1), so y = 3 * 0.7310585786300049 * 2."""
    spec = Spec(1, 1, score="sigmoid", weight="norm_sum")
    y = O.layer(np.array([[1.0]]), np.array([[0.3]], np.float32), None, spec,
                lambda e: (np.array([[1.0], [2.0]]), np.array([[3.0]])))
    assert abs(y[0, 0] - 4.386351471780029) < 1e-14


def test_ffn_all_experts_selected():
    """E = k: every token uses every expert, so y = sum_e w_e * FFN_e(x)."""
    spec, x, logits, bias, ge, gs = _small_layer(9, E=4, k=4, shared=0)
    spec.num_shared = 0
    y = O.layer(x, logits, bias, spec, ge)
    s = O.sigmoid(logits.astype(np.float64))
    w = 2.5 * s / s.sum(axis=1, keepdims=True)
    ref = sum(w[:, e:e + 1] * O.swiglu_expert(x, *ge(e)) for e in range(4))
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_ffn_linear_in_down_projection():
    spec, x, logits, bias, ge, gs = _small_layer(10, shared=0)
    spec.num_shared = 0
    y1 = O.layer(x, logits, bias, spec, ge)
    y3 = O.layer(x, logits, bias, spec, lambda e: (ge(e)[0], 3.0 * ge(e)[1]))
    assert np.allclose(y3, 3.0 * y1, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# E4M3 codec
# ---------------------------------------------------------------------------


def test_e4m3_decode_known_codes():
    g = _golden("e4m3_codes.json")
    for c, v in g["codes"].items():
        assert O.e4m3_decode(np.array([int(c)]))[0] == v
    assert np.isnan(O.e4m3_decode(np.array(g["nan_codes"]))).all()


def test_e4m3_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (127, 255)], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    back = O.e4m3_encode(vals)
    # +0 and -0 both encode to +0
    ok = (back == codes) | ((codes == 0x80) & (back == 0))
    assert ok.all()
    assert O.e4m3_encode(np.array([1000.0, -449.0, 448.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E]


def test_e4m3_ties_to_even():
    # halfway between 1.0 (0x38) and 1.125 (0x39) -> even 0x38;
    # halfway between 1.125 and 1.25 (0x3A) -> even 0x3A;
    # halfway between subnormals 2^-9 (0x01) and 2*2^-9 (0x02) -> 0x02
    v = np.array([1.0625, 1.1875, 1.5 * 2 ** -9, 0.5 * 2 ** -9], np.float32)
    assert O.e4m3_encode(v).tolist() == [0x38, 0x3A, 0x02, 0x00]


def test_quantize_rows_scales_and_grid_values():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    x[2, :128] = 0.0
    codes, scale = O.quantize_rows_1x128(x)
    assert scale.shape == (3, 2) and scale[2, 0] == 1.0
    assert (codes[2, :128] == 0).all()
    # the largest magnitude in each block maps to +-448
    for r in range(2):
        for b in range(2):
            blk = x[r, b * 128:(b + 1) * 128]
            assert scale[r, b] == np.float32(np.abs(blk).max()) / np.float32(448.0)
            j = np.argmax(np.abs(blk))
            assert O.e4m3_decode(codes[r, b * 128 + j]) * np.sign(blk[j]) == 448.0
    # values already on the grid times a power-of-two scale are exact
    grid = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    row = np.zeros((1, 128), np.float32)
    row[0, :127] = grid * 2.0 ** -3
    row[0, 126] = 448.0 * 2.0 ** -3
    c, s = O.quantize_rows_1x128(row)
    assert s[0, 0] == np.float32(2.0 ** -3)
    assert np.array_equal(O.e4m3_decode(c[0, :127]) * s[0, 0], row[0, :127])


def test_dequant_blocks():
    codes = np.full((128, 256), 0x38, np.uint8)  # 1.0
    scales = np.array([[0.5, 2.0]], np.float32)
    w = O.dequant_blocks(codes, scales)
    assert (w[:, :128] == 0.5).all() and (w[:, 128:] == 2.0).all()


# ---------------------------------------------------------------------------
# Load statistics
# ---------------------------------------------------------------------------


def test_imbalance_factor_exercise_3():
    g = _golden("imbalance_ex3.json")
    IF = O.imbalance_factor(g["tokens_per_expert"], g["G"])
    assert IF == g["imbalance_factor"]
    assert 1.0 - 1.0 / IF == g["wasted_fraction"]


def test_dispatch_bytes_per_token():
    """k * d_model * bytes ("The Two Costs"): DeepSeek-V3, bf16."""
    assert O.dispatch_bytes_per_token(8, 7168, 2) == 114688
    assert O.dispatch_bytes_per_token(8, 7168, 1) == 57344


def test_zipf_prefill_recipe_skew():
    """The prefill workload's bias must give hot experts above 5% of the
    assignments and leave some experts with none."""
    wl = mi.WORKLOADS["dsv3_prefill"]
    T = 4096
    idx, _, _ = O.route(mi.gen_logits(wl, T), mi.gen_bias(wl), wl)
    share = np.bincount(idx.reshape(-1), minlength=256) / (T * 8)
    assert share.max() > 0.05
    assert (share == 0).sum() >= 1


def test_gate_weights_do_not_depend_on_bias():
    """The bias steers which experts are chosen, never their weights: two
    biases that give the same selection give identical weights, and the
    weights are proportional to the sigmoid of the chosen logits."""
    wl = mi.WORKLOADS["dsv3"]
    logits = mi.gen_logits(wl, 128, seed=6)
    b = mi.gen_bias(wl, seed=6)
    idx1, w1, _ = O.route(logits, b, wl)
    idx2, w2, _ = O.route(logits, b + np.float32(0.25), wl)  # uniform shift: same order
    assert np.array_equal(idx1, idx2)
    assert np.array_equal(w1, w2)
    s = O.sigmoid(np.take_along_axis(logits.astype(np.float64), idx1, axis=1))
    assert np.allclose(w1 / w1[:, :1], s / s[:, :1], rtol=1e-13)


def test_fp8_path_dispatch_equals_dense_and_stays_close():
    """The E4M3 form of the layer: the dispatch-based path and the dense
    per-token path quantise the same rows the same way, so they agree; and
    quantising activations moves the output by a few percent at most."""
    rng = np.random.default_rng(12)
    E, k, d, F, T = 4, 2, 256, 128, 6
    spec = Spec(E, k, scale=2.5, shared=1)
    x = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    W13 = 0.05 * rng.standard_normal((E, 2 * F, d))
    W2 = 0.05 * rng.standard_normal((E, d, F))
    WS = (0.05 * rng.standard_normal((2 * F, d)), 0.05 * rng.standard_normal((d, F)))
    ge, gs = (lambda e: (W13[e], W2[e])), (lambda: WS)
    yq = O.layer(x, logits, None, spec, ge, gs, act_quant=True)
    y = O.layer(x, logits, None, spec, ge, gs)
    idx, w, _ = O.route(logits, None, spec)
    for t in range(T):
        assert np.allclose(yq[t], O.dense_token(x[t], idx[t], w[t], ge, gs, act_quant=True),
                           rtol=1e-12, atol=1e-12)
    rel = np.abs(yq - y).max() / np.abs(y).max()
    assert 0 < rel < 0.1


# ---------------------------------------------------------------------------
# router logits ([P2] moe_ep_layer listing: a linear map, then softmax/top-k)
# ---------------------------------------------------------------------------


def test_router_logits_special_cases():
    rng = np.random.default_rng(5)
    E, d = 6, 10
    wr = rng.standard_normal((E, d))
    # a one-hot token picks one column of the router weight, exactly
    for c in range(d):
        x = np.zeros((1, d))
        x[0, c] = 1.0
        assert np.array_equal(O.router_logits(x, wr)[0], wr[:, c])
    # zero tokens score zero
    assert np.array_equal(O.router_logits(np.zeros((3, d)), wr), np.zeros((3, E)))
    # identity router weights (E = d) hand the token back
    x = rng.standard_normal((4, d))
    assert np.array_equal(O.router_logits(x, np.eye(d)), x)


def test_route_from_hidden_state_with_identity_router():
    # with identity router weights, softmax routing from the hidden state takes
    # each token's k largest coordinates, in descending order
    rng = np.random.default_rng(6)
    spec = mi.WORKLOADS["qwen3"].with_(num_experts=16, top_k=3, d_model=16)
    x = rng.permuted(np.tile(np.arange(16, dtype=np.float64), (5, 1)), axis=1)
    logits = O.router_logits(x, np.eye(16)).astype(np.float32)
    idx, w, _ = O.route(logits, None, spec)
    for t in range(5):
        assert list(idx[t]) == list(np.argsort(-x[t], kind="stable")[:3])
        assert abs(w[t].sum() - 1.0) < 1e-12
