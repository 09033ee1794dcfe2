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
from oracle import moe_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(params=["numpy", "cpp"])
def orc(request):
    """The pins that exercise the layer run against both oracles: the numpy
    one (float64, one library primitive per step) and the plain C++ one
    (loops, double accumulation)."""
    return O if request.param == "numpy" else R


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
def test_expected_distinct_monte_carlo(orc, G, kg):
    """With zero bias and iid logits every expert is picked with probability
    k/E, also under group-limited routing (symmetry over experts and groups),
    so the mean number of distinct experts per batch of B tokens must match
    E(1 - (1 - k/E)^B) = 222.44 at (256, 8, 64).  2000 batches; the per-batch
    standard deviation is about 4.5, so the mean is good to about 0.1."""
    E, k, B, nb = 256, 8, 64, 2000
    spec = Spec(E, k, G, kg, score="sigmoid")
    logits = mi.normal_f32(11, 2, (nb * B, E), 1.0)
    idx, _, _ = orc.route(logits, np.zeros(E, np.float32), spec)
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
def test_route_matches_bruteforce(orc, case):
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
    idx, w, info = orc.route(logits, bias if score == "sigmoid" else None, spec)
    keys = info["keys"]
    for t in range(T):
        bf = _bruteforce_route([np.float32(v) for v in keys[t]], E, k, G, kg)
        assert list(idx[t]) == bf, (t, keys[t], idx[t], bf)


def test_selection_keys_precision_and_nan(orc):
    spec = Spec(4, 2)
    logits = np.array([[np.nan, 0.0, 1.0, -1.0]], np.float32)
    bias = np.array([0.0, 0.5, 0.0, 0.0], np.float32)
    keys = orc.selection_keys(logits, bias, "sigmoid")
    assert keys.dtype == np.float32
    assert keys[0, 0] == -np.inf
    assert keys[0, 1] == np.float32(0.5) + np.float32(0.5)
    assert keys[0, 2] == np.float32(1.0 / (1.0 + math.exp(-1.0)))
    idx, _, _ = orc.route(logits, bias, spec)
    assert list(idx[0]) == [1, 2]


def test_softmax_selection_equals_selection_on_probabilities(orc):
    """The moe_ep_layer listing selects on softmax probabilities; the oracle
    selects on logits.  Same order because softmax is strictly increasing."""
    spec = Spec(128, 8, score="softmax")
    logits = mi.gen_logits(mi.WORKLOADS["qwen3"], 512, seed=3)
    idx, _, _ = orc.route(logits, None, spec)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    ref = np.argsort(-p, axis=1, kind="stable")[:, :8]
    assert np.array_equal(idx, ref)


def test_softmax_weights_are_softmax_over_selected_logits(orc):
    spec = Spec(128, 8, score="softmax")
    logits = mi.gen_logits(mi.WORKLOADS["qwen3"], 64, seed=4)
    idx, w, _ = orc.route(logits, None, spec)
    sel = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-12, atol=1e-15)


def test_softmax_selected_weights_tiny_workload(orc):
    """Tiny workload: softmax over the two selected sigmoid scores."""
    wl = mi.WORKLOADS["tiny"]
    logits = mi.gen_logits(wl, 16)
    idx, w, _ = orc.route(logits, mi.gen_bias(wl), wl)
    s = O.sigmoid(np.take_along_axis(logits.astype(np.float64), idx, axis=1))
    ref = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-14)


@pytest.mark.parametrize("name", ["dsv3", "qwen3", "tiny", "dsv3_prefill"])
def test_route_invariants(orc, name):
    wl = mi.WORKLOADS[name]
    T = 256
    logits = mi.gen_logits(wl, T, seed=5)
    idx, w, info = orc.route(logits, mi.gen_bias(wl, seed=5), wl)
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
def test_dispatch_combine_inverse_permutation(orc, T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32).reshape(T, k)
    x = rng.standard_normal((T, 24)).astype(np.float32)
    counts, offsets, row_of, tok = orc.dispatch(idx, E)
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=E))
    assert counts.sum() == T * k and offsets[-1] == T * k
    # every row written exactly once
    assert sorted(row_of.reshape(-1).tolist()) == list(range(T * k))
    # rows of one expert are contiguous, ascending in token
    for e in range(E):
        toks = tok[offsets[e]:offsets[e + 1]]
        assert list(toks) == sorted(toks)
        assert all(e in idx[t] for t in toks)
    recv = orc.gather_rows(x.astype(np.float64), tok)
    for j0 in range(k):
        w = np.zeros((T, k))
        w[:, j0] = 1.0
        y = orc.combine(recv, row_of, w)
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
def test_ffn_dispatch_path_equals_dense_per_token(orc, seed):
    spec, x, logits, bias, ge, gs = _small_layer(seed, G=4 if seed % 2 else 1, kg=2 if seed % 2 else 1)
    y = orc.layer(x, logits, bias, spec, ge, gs)
    idx, w, _ = orc.route(logits, bias, spec)
    for t in range(x.shape[0]):
        yt = orc.dense_token(x[t], idx[t], w[t], ge, gs)
        assert np.allclose(y[t], yt, rtol=1e-12, atol=1e-12)


def test_ffn_zero_input_gives_zero(orc):
    spec, x, logits, bias, ge, gs = _small_layer(7)
    y = orc.layer(np.zeros_like(x), logits, bias, spec, ge, gs)
    assert np.array_equal(y, np.zeros_like(y))


def test_ffn_zero_up_projection_leaves_shared_only(orc):
    spec, x, logits, bias, ge, gs = _small_layer(8)
    F = 16

    def ge0(e):
        w13, w2 = ge(e)
        w13 = w13.copy()
        w13[F:] = 0.0
        return w13, w2
    y = orc.layer(x, logits, bias, spec, ge0, gs)
    ws13, ws2 = gs()
    Fs = ws13.shape[0] // 2
    g = x @ ws13[:Fs].T
    shared = (g / (1 + np.exp(-g)) * (x @ ws13[Fs:].T)) @ ws2.T
    assert np.allclose(y, shared, rtol=1e-13, atol=1e-13)


def test_ffn_scalar_case_by_hand(orc):
    """d = F = 1, one expert, k = 1: y = w * wd * silu(wg * x) * (wu * x).
    x = 1, wg = 1, wu = 2, wd = 3, w = 1: silu(1) = 0.7310585786300049 (the
    logistic function at 1), so y = 3 * 0.7310585786300049 * 2."""
    spec = Spec(1, 1, score="sigmoid", weight="norm_sum")
    y = orc.layer(np.array([[1.0]]), np.array([[0.3]], np.float32), None, spec,
                lambda e: (np.array([[1.0], [2.0]]), np.array([[3.0]])))
    assert abs(y[0, 0] - 4.386351471780029) < 1e-14


def test_ffn_all_experts_selected(orc):
    """E = k: every token uses every expert, so y = sum_e w_e * FFN_e(x)."""
    spec, x, logits, bias, ge, gs = _small_layer(9, E=4, k=4, shared=0)
    spec.num_shared = 0
    y = orc.layer(x, logits, bias, spec, ge)
    s = O.sigmoid(logits.astype(np.float64))
    w = 2.5 * s / s.sum(axis=1, keepdims=True)
    ref = sum(w[:, e:e + 1] * orc.swiglu_expert(x, *ge(e)) for e in range(4))
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_ffn_linear_in_down_projection(orc):
    spec, x, logits, bias, ge, gs = _small_layer(10, shared=0)
    spec.num_shared = 0
    y1 = orc.layer(x, logits, bias, spec, ge)
    y3 = orc.layer(x, logits, bias, spec, lambda e: (ge(e)[0], 3.0 * ge(e)[1]))
    assert np.allclose(y3, 3.0 * y1, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# E4M3 codec
# ---------------------------------------------------------------------------


def test_e4m3_decode_known_codes(orc):
    g = _golden("e4m3_codes.json")
    for c, v in g["codes"].items():
        assert orc.e4m3_decode(np.array([int(c)]))[0] == v
    assert np.isnan(orc.e4m3_decode(np.array(g["nan_codes"]))).all()


def test_e4m3_round_trip_and_saturation(orc):
    codes = np.array([c for c in range(256) if c not in (127, 255)], dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    back = orc.e4m3_encode(vals)
    # +0 and -0 both encode to +0
    ok = (back == codes) | ((codes == 0x80) & (back == 0))
    assert ok.all()
    assert orc.e4m3_encode(np.array([1000.0, -449.0, 448.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E]


def test_e4m3_ties_to_even(orc):
    # halfway between 1.0 (0x38) and 1.125 (0x39) -> even 0x38;
    # halfway between 1.125 and 1.25 (0x3A) -> even 0x3A;
    # halfway between subnormals 2^-9 (0x01) and 2*2^-9 (0x02) -> 0x02
    v = np.array([1.0625, 1.1875, 1.5 * 2 ** -9, 0.5 * 2 ** -9], np.float32)
    assert orc.e4m3_encode(v).tolist() == [0x38, 0x3A, 0x02, 0x00]


def test_quantize_rows_scales_and_grid_values(orc):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    x[2, :128] = 0.0
    codes, scale = orc.quantize_rows_1x128(x)
    assert scale.shape == (3, 2) and scale[2, 0] == 1.0
    assert (codes[2, :128] == 0).all()
    # the largest magnitude in each block maps to +-448
    for r in range(2):
        for b in range(2):
            blk = x[r, b * 128:(b + 1) * 128]
            assert scale[r, b] == np.float32(np.abs(blk).max()) / np.float32(448.0)
            j = np.argmax(np.abs(blk))
            assert orc.e4m3_decode(codes[r, b * 128 + j]) * np.sign(blk[j]) == 448.0
    # values already on the grid times a power-of-two scale are exact
    grid = orc.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    row = np.zeros((1, 128), np.float32)
    row[0, :127] = grid * 2.0 ** -3
    row[0, 126] = 448.0 * 2.0 ** -3
    c, s = orc.quantize_rows_1x128(row)
    assert s[0, 0] == np.float32(2.0 ** -3)
    assert np.array_equal(orc.e4m3_decode(c[0, :127]) * s[0, 0], row[0, :127])


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


def test_zipf_prefill_recipe_skew(orc):
    """The prefill workload's bias must give hot experts above 5% of the
    assignments and leave some experts with none."""
    wl = mi.WORKLOADS["dsv3_prefill"]
    T = 4096
    idx, _, _ = orc.route(mi.gen_logits(wl, T), mi.gen_bias(wl), wl)
    share = np.bincount(idx.reshape(-1), minlength=256) / (T * 8)
    assert share.max() > 0.05
    assert (share == 0).sum() >= 1


def test_gate_weights_do_not_depend_on_bias(orc):
    """The bias steers which experts are chosen, never their weights: two
    biases that give the same selection give identical weights, and the
    weights are proportional to the sigmoid of the chosen logits."""
    wl = mi.WORKLOADS["dsv3"]
    logits = mi.gen_logits(wl, 128, seed=6)
    b = mi.gen_bias(wl, seed=6)
    idx1, w1, _ = orc.route(logits, b, wl)
    idx2, w2, _ = orc.route(logits, b + np.float32(0.25), wl)  # uniform shift: same order
    assert np.array_equal(idx1, idx2)
    assert np.array_equal(w1, w2)
    s = O.sigmoid(np.take_along_axis(logits.astype(np.float64), idx1, axis=1))
    assert np.allclose(w1 / w1[:, :1], s / s[:, :1], rtol=1e-13)


def test_fp8_path_dispatch_equals_dense_and_stays_close(orc):
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
    yq = orc.layer(x, logits, None, spec, ge, gs, act_quant=True)
    y = orc.layer(x, logits, None, spec, ge, gs)
    idx, w, _ = orc.route(logits, None, spec)
    for t in range(T):
        assert np.allclose(yq[t], orc.dense_token(x[t], idx[t], w[t], ge, gs, act_quant=True),
                           rtol=1e-12, atol=1e-12)
    rel = np.abs(yq - y).max() / np.abs(y).max()
    assert 0 < rel < 0.1


# ---------------------------------------------------------------------------
# router logits ([P2] moe_ep_layer listing: a linear map, then softmax/top-k)
# ---------------------------------------------------------------------------


def test_router_logits_special_cases(orc):
    rng = np.random.default_rng(5)
    E, d = 6, 10
    wr = rng.standard_normal((E, d))
    # a one-hot token picks one column of the router weight, exactly
    for c in range(d):
        x = np.zeros((1, d))
        x[0, c] = 1.0
        assert np.array_equal(orc.router_logits(x, wr)[0], wr[:, c])
    # zero tokens score zero
    assert np.array_equal(orc.router_logits(np.zeros((3, d)), wr), np.zeros((3, E)))
    # identity router weights (E = d) hand the token back
    x = rng.standard_normal((4, d))
    assert np.array_equal(orc.router_logits(x, np.eye(d)), x)


def test_route_from_hidden_state_with_identity_router(orc):
    # with identity router weights, softmax routing from the hidden state takes
    # each token's k largest coordinates, in descending order
    rng = np.random.default_rng(6)
    spec = mi.WORKLOADS["qwen3"].with_(num_experts=16, top_k=3, d_model=16)
    x = rng.permuted(np.tile(np.arange(16, dtype=np.float64), (5, 1)), axis=1)
    logits = orc.router_logits(x, np.eye(16)).astype(np.float32)
    idx, w, _ = orc.route(logits, None, spec)
    for t in range(5):
        assert list(idx[t]) == list(np.argsort(-x[t], kind="stable")[:3])
        assert abs(w[t].sum() - 1.0) < 1e-12


# ---------------------------------------------------------------------------
# E4M3 activations inside the layer ("DeepEP" section, trick 1)
# ---------------------------------------------------------------------------


def _grid_layer(h_vals, x_scale=1.0):
    """One expert (E = k = 1, d = F = 128) whose token and SwiGLU activations
    are known exactly: x = x_scale * (1, 448, 0, ...); every gate row reads
    x[0] with weight 64 / x_scale, so gate = 64 and silu(64) = 64 in double
    (1 + e^-64 rounds to 1); up row i reads x[0] with weight h_i / (64 x_scale),
    so h_i is exactly the given value; W2 is the identity and the single
    weight is 1, so y = h."""
    d = F = 128
    h = np.zeros(F)
    h[:len(h_vals)] = h_vals
    x = np.zeros((1, d))
    x[0, 0], x[0, 1] = x_scale, 448.0 * x_scale
    w13 = np.zeros((2 * F, d))
    w13[:F, 0] = 64.0 / x_scale
    w13[F:, 0] = h / (64.0 * x_scale)
    w2 = np.eye(d)
    spec = Spec(1, 1)
    return spec, x, np.array([[0.3]], np.float32), (lambda e: (w13, w2)), h


@pytest.mark.parametrize("x_scale,h_scale", [(1.0, 1.0), (2.0 ** -3, 2.0 ** -5), (4.0, 2.0 ** 2)])
def test_act_quant_is_exact_on_the_grid(orc, x_scale, h_scale):
    """Activations that are E4M3 values times a power-of-two scale, with the
    block maximum at +-448 times that scale, quantise exactly: the quantised
    and the exact layer agree bit for bit, for x and for h."""
    grid = orc.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    vals = np.concatenate([grid[::-1][:64], -grid[1:64]]) * h_scale  # 448 * h_scale is the block max
    spec, x, logits, ge, h = _grid_layer(vals, x_scale)
    yq = orc.layer(x, logits, None, spec, ge, act_quant=True)
    y = orc.layer(x, logits, None, spec, ge)
    assert np.array_equal(y[0], h)
    assert np.array_equal(yq, y)


def test_act_quant_hand_computed_h_block(orc):
    """A 128-column block of h quantised by hand (tests/golden/e4m3_h_block.json):
    the quantised layer returns exactly the hand-derived dequantised values."""
    g = _golden("e4m3_h_block.json")
    spec, x, logits, ge, h = _grid_layer(np.array(g["h"]))
    yq = orc.layer(x, logits, None, spec, ge, act_quant=True)
    n = len(g["h"])
    assert yq[0, :n].tolist() == g["dequantised"]
    assert (yq[0, n:] == 0).all()
    codes, scales = orc.quantize_rows_1x128(h[None, :].astype(np.float32))
    assert codes[0, :n].tolist() == g["codes"]
    assert scales[0, 0] == np.float32(2.0 ** -7)


def test_softmax_selected_hand_computed(orc):
    g = _golden("softmax_selected.json")
    spec = Spec(4, 2, score="sigmoid", weight="softmax_selected")
    logits = np.array([g["logits"]], np.float32)
    idx, w, _ = orc.route(logits, np.zeros(4, np.float32), spec)
    assert idx[0].tolist() == g["idx"]
    assert np.abs(w[0] - np.array(g["weights"])).max() < g["tolerance"]


# ---------------------------------------------------------------------------
# Routing margins: how close a token's selection is to a tie
# ---------------------------------------------------------------------------


def _bruteforce_margin(keys, E, k, G, kg):
    """Smallest key difference between a selected and a non-selected eligible
    expert, and (grouped) between a chosen and a non-chosen group score, over
    all such pairs; NaN (infinite keys on both sides) counts as a tie (0)."""
    sel = _bruteforce_route(keys, E, k, G, kg)
    gsize = E // G
    gaps = []
    if G > 1:
        gscore = []
        for q in range(G):
            mem = list(range(q * gsize, (q + 1) * gsize))
            gscore.append(keys[mem[0]] if gsize == 1 else
                          max(np.float32(keys[a]) + np.float32(keys[b]) for a, b in itertools.combinations(mem, 2)))
        gscore = [np.float32(-np.inf) if np.isnan(v) else np.float32(v) for v in gscore]
        chosen = _lex_best(itertools.combinations(range(G), kg), gscore)
        gaps += [float(gscore[a]) - float(gscore[b]) for a in chosen for b in range(G) if b not in chosen]
        elig = [e for e in range(E) if e // gsize in chosen]
    else:
        elig = list(range(E))
    gaps += [float(keys[a]) - float(keys[b]) for a in sel for b in elig if b not in sel]
    gaps = [0.0 if np.isnan(v) else v for v in gaps]
    return min(gaps) if gaps else np.inf


@pytest.mark.parametrize("case", range(40))
def test_routing_margins_match_bruteforce(orc, case):
    rng = np.random.default_rng(2000 + case)
    E = int(rng.choice([4, 8, 12, 16]))
    G = int(rng.choice([g for g in (1, 2, 4) if E % g == 0]))
    kg = int(rng.integers(1, G + 1))
    k = min(int(rng.integers(1, kg * (E // G) + 1)), 6)
    T = 6
    logits = rng.choice(np.array([-1.0, -0.25, 0.0, 0.5, 2.0, 0.5001], np.float32), size=(T, E))
    if case % 4 == 0:
        logits[0, rng.integers(E)] = np.nan
        logits[1, :] = np.inf
        logits[2, rng.integers(E)] = -np.inf
        logits[3, :] = np.nan
    bias = rng.choice(np.array([0.0, 0.125, -0.125, 1e-6], np.float32), size=E)
    score = "softmax" if case % 3 == 0 else "sigmoid"
    spec = Spec(E, k, G, kg, score=score)
    b = bias if score == "sigmoid" else None
    idx, _, info = orc.route(logits, b, spec)
    gap = orc.routing_margins(info, spec)
    for t in range(T):
        ref = _bruteforce_margin([np.float32(v) for v in info["keys"][t]], E, k, G, kg)
        assert gap[t] == ref, (t, gap[t], ref)


def test_routing_margins_constructed_gaps(orc):
    """Softmax routing selects on the logits themselves, so the gaps are the
    logit differences: k-th vs (k+1)-th key, and group boundaries."""
    spec = Spec(8, 2, score="softmax")
    logits = np.array([[0.9, 0.5, 0.25, 0.0, -1, -1, -1, -1],      # gap 0.5 - 0.25
                       [0.9, 0.5, 0.5, 0.0, -1, -1, -1, -1],       # exact tie at the boundary
                       [3.0, 2.0, -np.inf, -np.inf, -np.inf, -np.inf, -np.inf, -np.inf]], np.float32)
    _, _, info = orc.route(logits, None, spec)
    gap = orc.routing_margins(info, spec)
    assert gap[0] == np.float64(np.float32(0.5)) - np.float64(np.float32(0.25))
    assert gap[1] == 0.0
    assert gap[2] == np.inf  # 2.0 against -inf
    # groups of two, keep one group: group scores 1.5 / 1.25 / ...: the group
    # boundary (0.25) is closer than the expert boundary inside the group
    spec = Spec(8, 1, G=4, kg=1, score="softmax")
    logits = np.array([[1.0, 0.5, 0.75, 0.5, -1, -1, -2, -2]], np.float32)
    _, _, info = orc.route(logits, None, spec)
    assert orc.routing_margins(info, spec)[0] == 0.25


# ---------------------------------------------------------------------------
# The two oracles agree on the workloads' own storage formats
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("name,T", [("tiny", 16), ("qwen3", 5), ("dsv3", 4), ("dsv3_fp8", 3)])
def test_cpp_oracle_reads_storage_formats_like_numpy(name, T):
    """The C++ oracle reads bf16 bits and E4M3 codes with block scales
    directly; the numpy oracle works on their float64 values.  Reduced widths,
    the workloads' routing rules, same seeded inputs: the two layers agree to
    rounding (different summation orders), and the E4M3 form with quantised
    activations as well."""
    wl = mi.WORKLOADS[name]
    if name != "tiny":
        wl = wl.with_(d_model=256, d_ff=128, d_ff_shared=256)
    x = mi.gen_x(wl, T, seed=3)
    logits = mi.gen_logits(wl, T, seed=3)
    bias = mi.gen_bias(wl, seed=3)
    E = wl.num_experts
    w13 = [mi.gen_weight(wl, "w13", e) for e in range(E)]
    w2 = [mi.gen_weight(wl, "w2", e) for e in range(E)]
    sh = (mi.gen_weight(wl, "ws13"), mi.gen_weight(wl, "ws2")) if wl.num_shared else None
    fp8 = wl.weight_dtype == "fp8"

    def f64(m):
        if fp8:
            return O.dequant_blocks(*m)
        return mi.bf16_bits_to_f32(m).astype(np.float64) if m.dtype == np.uint16 else m.astype(np.float64)
    xv = mi.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)
    ge = lambda e: (f64(w13[e]), f64(w2[e]))  # noqa: E731
    gs = (lambda: (f64(sh[0]), f64(sh[1]))) if sh else None
    for aq in ((False, True) if fp8 else (False,)):
        ref = O.layer(xv, logits, bias, wl, ge, gs, act_quant=aq)
        c = R.config(wl, d_model=wl.d_model, d_ff=wl.d_ff, d_ff_shared=wl.d_ff_shared,
                     act_dtype=wl.act_dtype, weight_dtype=wl.weight_dtype, act_quant=aq)
        cat = (lambda ms: np.ascontiguousarray(np.stack([m[0] if fp8 else m for m in ms])))
        cats = (lambda ms: np.ascontiguousarray(np.stack([m[1] for m in ms])))
        keep = [cat(w13), cat(w2), np.ascontiguousarray(x)]
        W = R.RefWeights(keep[0].ctypes.data, keep[1].ctypes.data, None, None, None, None, None, None)
        if fp8:
            keep += [cats(w13), cats(w2)]
            W.w13_scale, W.w2_scale = keep[3].ctypes.data, keep[4].ctypes.data
        if sh:
            s13, s2 = (np.ascontiguousarray(m[0] if fp8 else m) for m in sh)
            keep += [s13, s2]
            W.ws13, W.ws2 = s13.ctypes.data, s2.ctypes.data
            if fp8:
                t13, t2 = np.ascontiguousarray(sh[0][1]), np.ascontiguousarray(sh[1][1])
                keep += [t13, t2]
                W.ws13_scale, W.ws2_scale = t13.ctypes.data, t2.ctypes.data
        y = np.empty((T, wl.d_model))
        lg = np.ascontiguousarray(logits)
        bb = np.ascontiguousarray(bias) if bias is not None else None
        import ctypes
        st = R.lib().moe_ref_layer(ctypes.byref(c), T, keep[2].ctypes.data, lg.ctypes.data,
                                   bb.ctypes.data if bb is not None else None, ctypes.byref(W), None, None,
                                   y.ctypes.data, 2)
        assert st == 0
        assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max(), (aq, np.abs(y - ref).max())
