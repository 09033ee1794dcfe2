"""Plain CPU oracle of the expert-parallel MoE layer, one GPU's share.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (``combine_experts_amd``) never does, and this module imports
nothing from it.  It is written for a reader checking it against the pages,
not for speed: numpy in float64, one library primitive per step (a matrix
product, a sort), no blocking, fusion or reordering.

Sources (page title, then section):
  [P2]  "7.13 Serving Mixture-of-Experts: Expert Parallelism & All-to-All
        Inference" (llm-stack-book): "Why MoE Serving Is a Different Problem";
        "Expert Parallelism Mechanics: Dispatch, Compute, Combine" and its
        moe_ep_layer listing; "The Two Costs"; "DeepEP: A Production
        All-to-All Kernel"; "Hot-Expert Skew at Decode and Load Balancing";
        Exercises 2 and 3.
  [P3]  "One-Sided Expert-Parallel All-to-All for Mixture-of-Experts
        Inference over NVLink" (abstract of arXiv:2611.13188).
  [P4]  "Mixture-of-experts serving" (learn-kernels), paragraphs 1 and 4.

What is pinned, and how (tests/test_oracle_pins.py):
  router logits    one-hot tokens select one weight column; zero tokens give
                   zero logits; identity router weights give the token back;
                   with them, routing from the hidden state picks the token's
                   largest coordinates.
  route            brute-force enumeration on small E; invariants; the
                   expected-distinct-experts closed form of [P2] "Why MoE
                   Serving..." (Monte Carlo); softmax identity.
  dispatch/combine exact inverse permutation; counts = bincount.
  expert FFN       an independent dense per-token path; closed forms (x = 0,
                   zero up-projection, d = F = 1 by hand, E = k).
  routing margins  brute force over (selected, unselected) pairs; constructed gaps.
  e4m3 codec       values fixed by the OCP 8-bit floating point format
                   definition (max 448, subnormal step 2^-9), round trips,
                   saturation, ties to even.
  imbalance factor [P2] Exercise 3 table (IF = 2.0).
No page prints a layer output value; FFN numerics are pinned by the closed
forms and the independent dense formulation above, not by a printed number.

Readings where the pages are silent (each also listed in the design notes):
  * SwiGLU experts: silu(x Wg^T) * (x Wu^T), then W2.  The moe_ep_layer
    listing uses one up-projection and GELU; the layer built here is the
    DeepSeek-V3 / Qwen3 form.
  * Routing bias steers selection only; gate weights use unbiased scores
    ([P4] paragraph 1: the bias exists to keep load balanced).
  * Group-limited routing ([P4] paragraph 4 names it): contiguous groups of
    E / n_group experts, group score = sum of its two largest biased keys,
    keep the topk_group best groups, then top-k among their experts.
  * Ties go to the lower index (groups and experts); NaN keys count as -inf;
    experts outside the chosen groups are never selected.
  * Selection is decided on fp32 keys (the kernel's precision): sigmoid
    scores rounded to fp32, plus the fp32 bias, added in fp32.  Softmax
    routing selects on the fp32 logit, which orders experts exactly as the
    softmax probabilities of the moe_ep_layer listing do (softmax is strictly
    increasing in each logit).
  * Weights: normalised to sum 1 over the selected k, then multiplied by
    routed_scale.  The shared expert is never scaled.
  * fp8 (E4M3FN, max 448): per-token per-128-column activation scales
    amax/448 in fp32 (1 when amax = 0), code = nearest E4M3 value of x/scale
    in fp32 with ties to even, saturating at +-448.  Weights arrive as codes
    plus 128x128 block scales and mean code * scale.  The reference of the
    fp8 layer is the layer on those weights with exact activations
    (act_quant=False).  The "DeepEP" section quantises the dispatched rows
    only; the kernels also quantise h per 1x128 before the down GEMM, and
    act_quant=True reproduces that form (x, and h rounded to fp32, quantised)
    for a second, tighter comparison.

Also pinned: act_quant by closed forms (activations on the E4M3 grid times a
power-of-two scale quantise exactly; a hand-quantised 1x128 block of h), and
routing_margins by brute force over every (selected, unselected) pair.  A
plain C++ oracle (moe_ref.cpp) implements the same layer in loops; the pins
run against both.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# Routing: scores, group-limited top-k, gate weights
# ---------------------------------------------------------------------------


def sigmoid(z):
    """Sigmoid affinity in float64 ([P4] paragraph 1)."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def selection_keys(logits, bias, score):
    """fp32 selection keys [T][E].

    sigmoid: key = fp32(sigmoid(logit)) + bias   (fp32 add; bias may be None)
    softmax: key = logit (orders experts as the softmax probabilities do)
    NaN keys become -inf so every selected index stays in range."""
    logits = np.asarray(logits, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        if score == "sigmoid":
            key = sigmoid(logits).astype(np.float32)
            if bias is not None:
                key = key + np.asarray(bias, dtype=np.float32)[None, :]
        elif score == "softmax":
            key = logits.copy()
        else:
            raise ValueError(score)
    key = key.astype(np.float32)
    key[np.isnan(key)] = -np.inf
    return key


def group_scores(keys, n_group):
    """Group score [T][n_group]: fp32 sum of the two largest keys of each
    contiguous group of E / n_group experts (the largest one alone when a
    group holds a single expert)."""
    T, E = keys.shape
    g = keys.reshape(T, n_group, E // n_group)
    desc = -np.sort(-g, axis=2)
    if desc.shape[2] == 1:
        return desc[:, :, 0].astype(np.float32)
    with np.errstate(invalid="ignore"):
        s = (desc[:, :, 0] + desc[:, :, 1]).astype(np.float32)
    s[np.isnan(s)] = -np.inf  # (+inf) + (-inf) cannot occur after NaN->-inf, kept for safety
    return s


def ranked(values, eligible):
    """Indices of each row ordered by: eligible first, larger value first,
    lower index first (a stable sort)."""
    values = np.asarray(values)
    neg = -values.astype(np.float64)
    return np.lexsort((neg, ~eligible), axis=-1)


def choose_groups(gscores, topk_group):
    """Boolean [T][n_group]: the topk_group best groups per token."""
    T, G = gscores.shape
    order = ranked(gscores, np.ones((T, G), dtype=bool))
    chosen = np.zeros((T, G), dtype=bool)
    np.put_along_axis(chosen, order[:, :topk_group], True, axis=1)
    return chosen


def router_logits(x, w_router):
    """Router scores before the score function: logits[t][e] = x[t] . w_router[e].

    [P2] moe_ep_layer listing: the router is one linear map from the token to
    a score per expert; softmax and top-k (route below) follow.  Float64
    matrix product of the stored values."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def route(logits, bias, spec):
    """Router of one MoE layer for T tokens.

    [P2] moe_ep_layer listing (softmax, top-k, renormalise the chosen k) and
    [P4] paragraphs 1 and 4 (sigmoid affinity + per-expert bias, group-limited
    routing).  Returns (idx int32 [T][k] ordered by key, weights float64
    [T][k], info dict with keys, eligibility and group scores)."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    k, G, kg = spec.top_k, spec.n_group, spec.topk_group
    keys = selection_keys(logits, bias, spec.score)
    if G > 1:
        gs = group_scores(keys, G)
        chosen = choose_groups(gs, kg)
        eligible = np.repeat(chosen, E // G, axis=1)
    else:
        gs = None
        eligible = np.ones((T, E), dtype=bool)
    idx = ranked(keys, eligible)[:, :k].astype(np.int32)
    w = gate_weights(logits, idx, spec)
    return idx, w, {"keys": keys, "eligible": eligible, "group_scores": gs}


def gate_weights(logits, idx, spec):
    """Gate weights [T][k] in float64 from the unbiased scores of the chosen
    experts, normalised over the k, then times routed_scale."""
    logits64 = np.asarray(logits, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        if spec.score == "softmax":
            # softmax over all experts, then keep and renormalise the chosen k
            m = np.max(logits64, axis=1, keepdims=True)
            p = np.exp(logits64 - m)
            p = p / p.sum(axis=1, keepdims=True)
            sel = np.take_along_axis(p, idx, axis=1)
        else:
            sel = np.take_along_axis(sigmoid(logits64), idx, axis=1)
        if spec.weight == "norm_sum":
            w = sel / sel.sum(axis=1, keepdims=True)
        elif spec.weight == "softmax_selected":
            ex = np.exp(sel - sel.max(axis=1, keepdims=True))
            w = ex / ex.sum(axis=1, keepdims=True)
        else:
            raise ValueError(spec.weight)
    return w * float(spec.routed_scale)


def routing_margins(info, spec):
    """Per-token closeness of the selection to a tie: the gap between the
    k-th and (k+1)-th eligible keys, and (grouped routing) the gap between the
    topk_group-th and next group scores.  A GPU choice may differ from the
    oracle only where the smaller gap is within the stated tolerance."""
    keys, elig = info["keys"].astype(np.float64), info["eligible"]
    k = spec.top_k
    T, E = keys.shape
    order = ranked(keys, elig)
    kth = np.take_along_axis(keys, order[:, k - 1:k], axis=1)[:, 0]
    has_next = elig.sum(axis=1) > k
    if E > k:
        nxt = np.take_along_axis(keys, order[:, k:k + 1], axis=1)[:, 0]
        with np.errstate(invalid="ignore"):
            gap = np.where(has_next, kth - nxt, np.inf)
    else:
        gap = np.full(T, np.inf)
    gs = info["group_scores"]
    if gs is not None and spec.topk_group < gs.shape[1]:
        g64 = gs.astype(np.float64)
        gord = ranked(g64, np.ones_like(g64, dtype=bool))
        a = np.take_along_axis(g64, gord[:, spec.topk_group - 1:spec.topk_group], axis=1)[:, 0]
        b = np.take_along_axis(g64, gord[:, spec.topk_group:spec.topk_group + 1], axis=1)[:, 0]
        with np.errstate(invalid="ignore"):
            gap = np.minimum(gap, a - b)
    gap = np.where(np.isnan(gap), 0.0, gap)
    return gap


# ---------------------------------------------------------------------------
# Dispatch and combine
# ---------------------------------------------------------------------------


def dispatch(idx, num_experts):
    """Canonical dispatch layout ([P2] "Expert Parallelism Mechanics", step 2:
    rows of the same expert contiguous; [P3]: expert-grouped receive buffer).

    Rows of expert e occupy [offset[e], offset[e+1]) in ascending token order.
    Returns counts [E], offsets [E+1], row_of [T][k], token_of_row [T*k]."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=num_experts).astype(np.int64)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_of = np.full((T, k), -1, dtype=np.int64)
    token_of_row = np.full(T * k, -1, dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            r = fill[e]
            fill[e] += 1
            row_of[t, j] = r
            token_of_row[r] = t
    return counts, offsets, row_of, token_of_row


def gather_rows(x, token_of_row):
    """recv[row] = x[token of row] (the dispatch payload)."""
    return np.asarray(x)[token_of_row]


def combine(expert_out, row_of, w, shared_out=None):
    """y[t] = shared_out[t] + sum_j w[t][j] * expert_out[row_of[t][j]]
    ([P2] moe_ep_layer listing: weighted scatter-add back to the home token;
    DeepEP sketch: combine(...) + shared_out)."""
    T, k = row_of.shape
    y = np.zeros((T, expert_out.shape[1]), dtype=np.float64)
    for j in range(k):
        y += np.asarray(w, dtype=np.float64)[:, j:j + 1] * expert_out[row_of[:, j]]
    if shared_out is not None:
        y += shared_out
    return y


# ---------------------------------------------------------------------------
# Expert FFN (SwiGLU)
# ---------------------------------------------------------------------------


def silu(z):
    return z * sigmoid(z)


def swiglu_expert(a, w13, w2, act_quant=False):
    """One expert on rows a [n][d]: w13 [2F][d] holds gate rows [0, F) and up
    rows [F, 2F); w2 is [d][F].  out = (silu(a Wg^T) * (a Wu^T)) W2^T.

    act_quant: the quantised-activation form of the E4M3 kernels ("DeepEP"
    section, trick 1, quantises the dispatched rows; the kernels also
    quantise h): the rows entering each GEMM are first quantised per 1x128
    block (the input rows as fp32, h after rounding to fp32) and the GEMM
    reads their dequantised values code * scale."""
    a = np.asarray(a, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    F = w13.shape[0] // 2
    if act_quant:
        a = dequant_rows_1x128(*quantize_rows_1x128(a.astype(np.float32)))
    gate = a @ w13[:F].T
    up = a @ w13[F:].T
    h = silu(gate) * up
    if act_quant:
        h = dequant_rows_1x128(*quantize_rows_1x128(h.astype(np.float32)))
    return h @ w2.T


def expert_ffn(recv, offsets, get_expert, act_quant=False):
    """Grouped expert compute over the dispatched rows ([P2] step 3: one
    matmul per expert); get_expert(e) -> (w13, w2) as float64."""
    recv = np.asarray(recv, dtype=np.float64)
    out = None
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        w13, w2 = get_expert(e)
        o = swiglu_expert(recv[lo:hi], w13, w2, act_quant)
        if out is None:
            out = np.zeros((recv.shape[0], o.shape[1]), dtype=np.float64)
        out[lo:hi] = o
    return out


def layer(x, logits, bias, spec, get_expert, get_shared=None, idx=None, w=None, act_quant=False):
    """The whole layer, step by step: route, dispatch, expert FFN, shared
    expert, combine.  Passing idx and w evaluates the layer under a given
    routing (used where a near-tie legitimately flips a choice)."""
    x = np.asarray(x, dtype=np.float64)
    if idx is None:
        idx, w, _ = route(logits, bias, spec)
    counts, offsets, row_of, token_of_row = dispatch(idx, spec.num_experts)
    recv = gather_rows(x, token_of_row)
    out = expert_ffn(recv, offsets, get_expert, act_quant)
    shared = None
    if spec.num_shared and get_shared is not None:
        ws13, ws2 = get_shared()
        shared = swiglu_expert(x, ws13, ws2, act_quant)
    return combine(out, row_of, w, shared)


def dense_token(x_t, idx_t, w_t, get_expert, get_shared=None, act_quant=False):
    """Brute-force output of one token: loop over its k experts and the shared
    expert directly from x and the weights, never touching a dispatch buffer.
    act_quant as in swiglu_expert, applied to this token's row alone."""
    x_t = np.asarray(x_t, dtype=np.float64)
    if act_quant:
        x_t = dequant_rows_1x128(*quantize_rows_1x128(x_t[None, :].astype(np.float32)))[0]

    def one(w13, w2):
        w13 = np.asarray(w13, dtype=np.float64)
        F = w13.shape[0] // 2
        g = np.array([np.dot(w13[i], x_t) for i in range(F)])
        u = np.array([np.dot(w13[F + i], x_t) for i in range(F)])
        h = g / (1.0 + np.exp(-g)) * u
        if act_quant:
            h = dequant_rows_1x128(*quantize_rows_1x128(h[None, :].astype(np.float32)))[0]
        return np.asarray(w2, dtype=np.float64) @ h

    y = np.zeros(x_t.shape[0], dtype=np.float64)
    for j in range(len(idx_t)):
        y += float(w_t[j]) * one(*get_expert(int(idx_t[j])))
    if get_shared is not None:
        y += one(*get_shared())
    return y


# ---------------------------------------------------------------------------
# fp8 E4M3FN ([P2] "DeepEP", trick 1: activations quantised to E4M3)
# ---------------------------------------------------------------------------


def e4m3_decode(codes):
    """Value of E4M3FN codes: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_decode(np.arange(127))  # finite non-negative codes 0..126


def e4m3_encode(v32):
    """Nearest E4M3FN code of fp32 values (ties to the even code), saturating
    to +-448; found by comparing against every finite code."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    a = np.abs(v).reshape(-1)
    d = np.abs(a[:, None] - _E4M3_POS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes (at most two, adjacent) take the even one
    even = cand & ((np.arange(127)[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a >= E4M3_MAX, 126, pick)
    code = pick.astype(np.int64)
    code = np.where((v.reshape(-1) < 0) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8).reshape(np.shape(v32))


def quantize_rows_1x128(x32):
    """Per-token, per-128-column E4M3 quantisation of fp32 rows [n][d]:
    scale = amax / 448 in fp32 (1 when amax = 0), code = e4m3(x / scale) with
    the division in fp32.  Returns (codes [n][d], scales [n][d/128])."""
    x32 = np.asarray(x32, dtype=np.float32)
    n, d = x32.shape
    blocks = x32.reshape(n, d // 128, 128)
    amax = np.abs(blocks).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (blocks / scale[:, :, None]).astype(np.float32)
    return e4m3_encode(q).reshape(n, d), scale


def dequant_rows_1x128(codes, scales):
    """Values code * scale of per-row, per-128-column quantised rows."""
    return e4m3_decode(codes) * np.repeat(np.asarray(scales, dtype=np.float64), 128, axis=1)


def dequant_blocks(codes, scales, block=128):
    """Weights from codes [rows][cols] and [rows/128][cols/128] block scales."""
    v = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, dtype=np.float64), block, axis=0), block, axis=1)
    return v * s


# ---------------------------------------------------------------------------
# Closed forms and load statistics
# ---------------------------------------------------------------------------


def expected_distinct(E, k, B):
    """Expected number of distinct experts touched by B tokens each picking k
    of E uniformly ([P2] "Why MoE Serving Is a Different Problem")."""
    return E * (1.0 - (1.0 - k / E) ** B)


def imbalance_factor(counts, G):
    """max over ranks of the rank load / mean rank load, experts laid out
    contiguously over G ranks ([P2] "Hot-Expert Skew", Exercise 3)."""
    c = np.asarray(counts, dtype=np.float64)
    loads = c.reshape(G, -1).sum(axis=1)
    return loads.max() / loads.mean()


def dispatch_bytes_per_token(k, d_model, bytes_per_elem):
    """All-to-all bytes per token per layer per direction, about
    k * d_model * bytes ([P2] "The Two Costs")."""
    return k * d_model * bytes_per_elem
