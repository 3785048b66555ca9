"""Pins for the oracle: checks against things other than the oracle itself.

Every pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix. They are kept here (not in a test_ file) so that the
same suite runs against the real oracle (test_oracle_pins.py) and against builds of it with a
planted mistake (test_oracle_mutants.py), which each pin set must catch.

What pins what:
  * top-k order: a full stable library sort (numpy lexsort), brute-force ranks on tiny rows,
    hand-built ties (boundary ties, +0/-0), shift invariance;
  * logsumexp / unary: exp(x - lse) sums to 1, scipy's logsumexp, scipy's softmax at the
    candidates, the constant-row closed form (lse = c + ln V);
  * gate: numpy matmul, one-hot hidden rows select rows of W_sel, W_sel = 0;
  * lattice: an identity gate reduces the pairwise term to a plain matmul, one-hot codebooks
    give a closed form that fixes the predecessor/successor roles, the anchor and the indices,
    zero codebooks leave the unary term, linearity in the gate;
  * walk: exhaustive enumeration of all k^L index paths (lexicographic greedy order), path
    score = sum of the chosen edges, margins from a sorted row, exact edge ties go to the lower
    index, and reduction to the per-position argmax of the logits (plain DFlash) for k = 1, zero
    codebooks and a zero gate;
  * sampling walk: stratified uniforms reproduce softmax(e / T) (scipy) to one stratum, a tiny
    temperature reproduces the greedy walk, the draw follows the chosen predecessor, closed-form
    draws and confidences on a two-candidate row;
  * p_min stop: closed-form confidences 1 / (1 + e^-d) and the resulting block lengths, a
    confidence exactly at p_min, k = 1;
  * dynamic convolution: with a zero dynamic part, numpy's convolve per channel; the impulse
    response (taps, the coefficient of the output row); block locality; the group broadcast;
  * LM-head top-k: the logits equal numpy's matmul of hidden with W_lm transposed, and the ids,
    unary and lse equal a stable sort and scipy's logsumexp of those logits; one-hot W_lm rows
    give logits x[i][v] = c_v * hidden[i][h(v)]; a zero hidden row gives lse = ln V.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import scipy.special

F32, BF16 = 0, 1


def bf16_bits(x) -> np.ndarray:
    """float32 values that are exactly representable in bf16 -> their bf16 bits."""
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def widen(a: np.ndarray) -> np.ndarray:
    """Stored tensor -> float64 (bf16 bits via numpy's own bit reinterpretation)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sort_order(row: np.ndarray) -> np.ndarray:
    """All token ids by (logit descending, id ascending), via numpy's stable lexsort."""
    ids = np.arange(row.size)
    return np.lexsort((ids, -row))


def _logit_cases():
    rng = np.random.default_rng(12345)
    cases = []
    cases.append((rng.normal(0, 3, (6, 777)).astype(np.float32), 5))
    cases.append((rng.integers(-3, 4, (8, 300)).astype(np.float32), 7))          # heavy ties
    x = rng.integers(-2, 3, (5, 64)).astype(np.float32)
    x[x == 0] = np.where(rng.random((x == 0).sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    cases.append((x, 33))                                                       # +0/-0 mix
    cases.append((rng.normal(0, 1, (3, 50)).astype(np.float32), 50))            # k = V
    cases.append((rng.normal(0, 3, (4, 1021)).astype(np.float32), 1))           # k = 1
    xb = rng.normal(0, 3, (4, 2048)).astype(np.float32)
    xb = (xb.view(np.uint32) & 0xFFFF0000).view(np.float32)                     # bf16-exact
    cases.append((bf16_bits(xb), 16))
    xt = np.round(rng.normal(0, 2, (4, 513)) * 4).astype(np.float32) / 4        # ties in bf16
    cases.append((bf16_bits(xt), 20))
    return cases


# ---------------------------------------------------------------------------------- top-k

def pin_topk_full_sort(o):
    for logits, k in _logit_cases():
        ids, unary, lse = o.topk_lse(logits, k)
        x = widen(logits)
        for row in range(x.shape[0]):
            want = sort_order(x[row])[:k]
            assert np.array_equal(ids[row], want), f"top-{k} differs from a full sort (row {row})"
            assert np.all(np.diff(unary[row]) <= 0), "unary not in candidate order"


def pin_topk_bruteforce_rank(o):
    rng = np.random.default_rng(7)
    for trial in range(6):
        V = 9
        x = rng.integers(-2, 3, (1, V)).astype(np.float32)
        for k in range(1, V + 1):
            ids, _, _ = o.topk_lse(x, k)
            rank = [sum(1 for u in range(V) if x[0, u] > x[0, v] or (x[0, u] == x[0, v] and u < v))
                    for v in range(V)]
            want = [rank.index(j) for j in range(k)]
            assert list(ids[0]) == want, f"brute-force ranks disagree (k={k}, trial {trial})"


def pin_topk_boundary_ties(o):
    # tokens 3, 8, 11 share the k-th value; the lowest ids win the remaining places
    x = np.full((1, 16), -5.0, np.float32)
    x[0, [2, 14]] = 7.0
    x[0, [11, 3, 8]] = 2.0
    ids, _, _ = o.topk_lse(x, 4)
    assert list(ids[0]) == [2, 14, 3, 8]
    # equal values at the top are ordered by id
    x = np.zeros((1, 6), np.float32)
    x[0, [5, 1]] = 1.0
    ids, _, _ = o.topk_lse(x, 3)
    assert list(ids[0]) == [1, 5, 0]


def pin_topk_signed_zero(o):
    x = np.full((1, 8), -1.0, np.float32)
    x[0, 2] = -0.0
    x[0, 5] = 0.0
    ids, unary, _ = o.topk_lse(x, 2)
    assert list(ids[0]) == [2, 5], "+0 and -0 are one value; the lower id comes first"
    assert unary[0, 0] == unary[0, 1]
    x[0, 2], x[0, 5] = 0.0, -0.0
    ids, _, _ = o.topk_lse(x, 2)
    assert list(ids[0]) == [2, 5]


def pin_topk_shift_invariance(o):
    rng = np.random.default_rng(3)
    x = rng.integers(-20, 21, (4, 400)).astype(np.float32)
    ids0, u0, l0 = o.topk_lse(x, 9)
    ids1, u1, l1 = o.topk_lse(x + np.float32(64.0), 9)
    assert np.array_equal(ids0, ids1)
    assert np.allclose(u0, u1, rtol=0, atol=1e-12)
    assert np.allclose(l1 - l0, 64.0, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------- logsumexp / unary

def pin_lse_normalises(o):
    for logits, k in _logit_cases():
        _, _, lse = o.topk_lse(logits, k)
        x = widen(logits)
        for row in range(x.shape[0]):
            total = math.fsum(np.exp(x[row] - lse[row]))
            assert abs(total - 1.0) < 1e-12, f"exp(x - lse) sums to {total!r}"


def pin_lse_scipy(o):
    for logits, k in _logit_cases():
        _, _, lse = o.topk_lse(logits, k)
        want = scipy.special.logsumexp(widen(logits), axis=1)
        assert np.allclose(lse, want, rtol=1e-13, atol=1e-13)


def pin_unary_softmax(o):
    for logits, k in _logit_cases():
        ids, unary, _ = o.topk_lse(logits, k)
        sm = scipy.special.softmax(widen(logits), axis=1)
        for row in range(ids.shape[0]):
            assert np.allclose(np.exp(unary[row]), sm[row, ids[row]], rtol=1e-12, atol=0)


def pin_constant_row(o):
    for V, k in [(1024, 4), (151, 151), (7, 1)]:
        x = np.full((2, V), 2.5, np.float32)
        ids, unary, lse = o.topk_lse(x, k)
        assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (2, 1)))
        assert np.allclose(lse, 2.5 + math.log(V), rtol=0, atol=1e-12)
        assert np.allclose(unary, -math.log(V), rtol=0, atol=1e-12)


def pin_bf16_values(o):
    vals = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 6.0, -1.0e-3, 12.0], np.float32)
    vals = (vals.view(np.uint32) & 0xFFFF0000).view(np.float32)
    ids, unary, lse = o.topk_lse(bf16_bits(vals)[None, :], 8)
    import torch
    widened = torch.tensor(bf16_bits(vals).view(np.int16)).view(torch.bfloat16).double().numpy()
    want_lse = scipy.special.logsumexp(widened)
    assert np.allclose(lse[0], want_lse, rtol=1e-14, atol=0)
    assert list(ids[0]) == list(sort_order(widened))
    assert np.allclose(unary[0], widened[ids[0]] - want_lse, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------------- gate

def pin_gate_matmul(o):
    rng = np.random.default_rng(11)
    for R, H, r, bf in [(5, 37, 16, False), (16, 256, 64, True), (3, 8, 3, True)]:
        h = rng.normal(0, 1, (R, H)).astype(np.float32)
        w = (rng.normal(0, 1, (H, r)) / math.sqrt(H)).astype(np.float32)
        if bf:
            h = (h.view(np.uint32) & 0xFFFF0000).view(np.float32)
            w = (w.view(np.uint32) & 0xFFFF0000).view(np.float32)
            g = o.gate(bf16_bits(h), bf16_bits(w))
        else:
            g = o.gate(h, w)
        want = h.astype(np.float64) @ w.astype(np.float64)
        scale = np.abs(h.astype(np.float64)) @ np.abs(w.astype(np.float64))
        assert np.all(np.abs(g - want) <= 1e-13 * scale + 1e-300)


def pin_gate_onehot_rows(o):
    rng = np.random.default_rng(5)
    for H, r in [(6, 4), (5, 5), (3, 9)]:
        w = rng.normal(0, 1, (H, r)).astype(np.float32)
        g = o.gate(np.eye(H, dtype=np.float32), w)
        assert np.array_equal(g, w.astype(np.float64)), "one-hot hidden row h must select W_sel[h]"


def pin_gate_zero(o):
    rng = np.random.default_rng(6)
    g = o.gate(rng.normal(0, 1, (4, 32)).astype(np.float32), np.zeros((32, 8), np.float32))
    assert np.all(g == 0.0)


# -------------------------------------------------------------------------------- lattice

def _lattice_inputs(rng, B, L, V, k, r):
    cand = np.stack([np.stack([rng.choice(V, k, replace=False) for _ in range(L)])
                     for _ in range(B)]).astype(np.int32)
    unary = rng.normal(-5, 2, (B, L, k))
    g = rng.normal(0, 1, (B, L, r))
    anchor = rng.integers(0, V, B).astype(np.int32)
    return cand, unary, g, anchor


def pin_lattice_identity_gate(o):
    rng = np.random.default_rng(21)
    B, L, V, k, r = 2, 3, 40, 5, 6
    cand, unary, _, anchor = _lattice_inputs(rng, B, L, V, k, r)
    pred = rng.normal(0, 1, (V, r)).astype(np.float32)
    succ = rng.normal(0, 1, (V, r)).astype(np.float32)
    edges = o.lattice(cand, unary, np.ones((B, L, r)), pred, succ, anchor)
    P, S = pred.astype(np.float64), succ.astype(np.float64)
    for b in range(B):
        for p in range(L):
            prev = np.full(k, anchor[b]) if p == 0 else cand[b, p - 1]
            want = unary[b, p][None, :] + P[prev] @ S[cand[b, p]].T
            assert np.allclose(edges[b, p], want, rtol=1e-13, atol=1e-13)


def pin_lattice_onehot_codes(o):
    rng = np.random.default_rng(22)
    B, L, V, k, r = 3, 4, 12, 4, 3
    cand, unary, g, anchor = _lattice_inputs(rng, B, L, V, k, r)
    code_p = rng.integers(0, r, V)
    code_s = rng.integers(0, r, V)
    pred = np.eye(r, dtype=np.float32)[code_p]
    succ = np.eye(r, dtype=np.float32)[code_s]
    edges = o.lattice(cand, unary, g, pred, succ, anchor)
    for b in range(B):
        for p in range(L):
            for i in range(k):
                prev = anchor[b] if p == 0 else cand[b, p - 1, i]
                for j in range(k):
                    match = code_p[prev] == code_s[cand[b, p, j]]
                    want = unary[b, p, j] + (g[b, p, code_p[prev]] if match else 0.0)
                    assert edges[b, p, i, j] == want, (b, p, i, j)


def pin_lattice_zero_codebooks(o):
    rng = np.random.default_rng(23)
    B, L, V, k, r = 2, 3, 30, 6, 8
    cand, unary, g, anchor = _lattice_inputs(rng, B, L, V, k, r)
    z = np.zeros((V, r), np.float32)
    edges = o.lattice(cand, unary, g, z, z, anchor)
    assert np.array_equal(edges, np.broadcast_to(unary[:, :, None, :], edges.shape))


def pin_lattice_linear_in_gate(o):
    rng = np.random.default_rng(24)
    B, L, V, k, r = 2, 3, 50, 5, 7
    cand, unary, g1, anchor = _lattice_inputs(rng, B, L, V, k, r)
    g2 = rng.normal(0, 1, g1.shape)
    pred = rng.normal(0, 1, (V, r)).astype(np.float32)
    succ = rng.normal(0, 1, (V, r)).astype(np.float32)
    pair = lambda g: o.lattice(cand, unary, g, pred, succ, anchor) - unary[:, :, None, :]
    assert np.allclose(pair(g1 + g2), pair(g1) + pair(g2), rtol=1e-12, atol=1e-12)
    assert np.allclose(pair(2.0 * g1), 2.0 * pair(g1), rtol=1e-12, atol=1e-12)
    assert np.all(pair(np.zeros_like(g1)) == 0.0)


def pin_lattice_anchor_rows(o):
    rng = np.random.default_rng(25)
    B, L, V, k, r = 3, 2, 64, 8, 16
    cand, unary, g, anchor = _lattice_inputs(rng, B, L, V, k, r)
    pred = rng.normal(0, 1, (V, r)).astype(np.float32)
    succ = rng.normal(0, 1, (V, r)).astype(np.float32)
    edges = o.lattice(cand, unary, g, pred, succ, anchor)
    for b in range(B):
        assert np.all(edges[b, 0] == edges[b, 0, 0][None, :]), "position 0 rows must be equal"


# ----------------------------------------------------------------------------------- walk

def _walk_cases():
    rng = np.random.default_rng(31)
    out = []
    for B, L, k in [(2, 4, 4), (3, 3, 5), (1, 5, 3), (2, 2, 1)]:
        edges = rng.integers(-3, 4, (B, L, k, k)).astype(np.float64)   # many exact ties
        edges[:, 0] = edges[:, 0, :1]                                  # position 0 rows equal
        cand = rng.integers(0, 1000, (B, L, k)).astype(np.int32)
        out.append((edges, cand))
    e = rng.normal(0, 1, (2, 4, 4, 4))
    e[:, 0] = e[:, 0, :1]
    out.append((e, rng.integers(0, 1000, (2, 4, 4)).astype(np.int32)))
    return out


def pin_walk_bruteforce(o):
    for edges, cand in _walk_cases():
        B, L, k = cand.shape
        path, idx, _, _ = o.walk(edges, cand)
        for b in range(B):
            best_key, best = None, None
            for js in itertools.product(range(k), repeat=L):
                key, prev = [], 0
                for p, j in enumerate(js):
                    key += [-edges[b, p, prev, j], j]
                    prev = j
                if best_key is None or key < best_key:
                    best_key, best = key, js
            assert tuple(idx[b]) == best, f"walk {tuple(idx[b])} vs enumeration {best}"
            assert np.array_equal(path[b], cand[b, np.arange(L), list(best)])


def pin_walk_score_and_margin(o):
    for edges, cand in _walk_cases():
        B, L, k = cand.shape
        _, idx, margin, score = o.walk(edges, cand)
        for b in range(B):
            prev, chosen = 0, []
            for p in range(L):
                row = np.sort(edges[b, p, prev])
                chosen.append(edges[b, p, prev, idx[b, p]])
                want = math.inf if k == 1 else row[-1] - row[-2]
                assert margin[b, p] == want
                prev = idx[b, p]
            assert abs(score[b] - math.fsum(chosen)) <= 1e-12 * max(1.0, abs(score[b]))


def pin_walk_edge_tie(o):
    # tokens 5 and 9 share the top logit and the successor code: every lattice row has an exact
    # tie between candidate 0 (token 5) and candidate 1 (token 9); the walk takes index 0
    V, r = 16, 4
    rng = np.random.default_rng(41)
    logits = np.full((1, 3, V), -3.0, np.float32)
    logits[0, :, 5] = 4.0
    logits[0, :, 9] = 4.0
    hidden = rng.normal(0, 1, (1, 3, 8)).astype(np.float32)
    W = rng.normal(0, 1, (8, r)).astype(np.float32)
    pred = rng.normal(0, 1, (V, r)).astype(np.float32)
    succ = rng.normal(0, 1, (V, r)).astype(np.float32)
    succ[9] = succ[5]
    res = o.select(logits, hidden, W, pred, succ, np.array([2], np.int32), 3)
    assert np.array_equal(res.cand_ids[0, :, :2], np.tile([5, 9], (3, 1)))
    assert np.all(res.edges[0, :, :, 0] == res.edges[0, :, :, 1])
    assert list(res.path[0]) == [5, 5, 5] and np.all(res.margin[0] == 0.0)


def _argmax_reduction_inputs(seed):
    rng = np.random.default_rng(seed)
    B, L, V, H, r = 3, 4, 200, 16, 8
    logits = rng.normal(0, 3, (B, L, V)).astype(np.float32)
    logits[0, 1, [17, 40]] = logits[0, 1].max() + 1.0   # exact tie at the top: lowest id wins
    hidden = rng.normal(0, 1, (B, L, H)).astype(np.float32)
    W = rng.normal(0, 1, (H, r)).astype(np.float32)
    pred = rng.normal(0, 1, (V, r)).astype(np.float32)
    succ = rng.normal(0, 1, (V, r)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    return logits, hidden, W, pred, succ, anchor


def pin_reduces_to_argmax(o):
    logits, hidden, W, pred, succ, anchor = _argmax_reduction_inputs(51)
    want = np.argmax(logits, axis=2)   # first maximum = lowest id
    z_cb = np.zeros_like(pred)
    for args, k in [((hidden, W, pred, succ), 1),                    # k = 1
                    ((hidden, W, z_cb, z_cb), 5),                    # zero codebooks
                    ((hidden, np.zeros_like(W), pred, succ), 5),     # zero gate weight
                    ((np.zeros_like(hidden), W, pred, succ), 5)]:    # zero hidden state
        res = o.select(logits, *args, anchor, k)
        assert np.array_equal(res.path, want), f"no reduction to argmax (k={k})"


# ---------------------------------------------------- walk modes: sampling and the p_min stop

def pin_sample_frequencies(o):
    # one position, identical rows, stratified uniforms u_i = (i + 1/2) / N: the share of each
    # index equals softmax(e / T) up to one stratum (closed form via scipy's softmax)
    rng = np.random.default_rng(61)
    N, k = 4000, 5
    e = rng.normal(0, 1.5, k)
    edges = np.broadcast_to(e, (N, 1, k, k)).copy()
    cand = np.broadcast_to(np.arange(100, 100 + k, dtype=np.int32), (N, 1, k)).copy()
    u = ((np.arange(N) + 0.5) / N).reshape(N, 1)
    for T in (0.5, 1.0, 2.0):
        _, idx, _, _, _ = o.walk_ex(edges, cand, T, u, 0.0)
        share = np.bincount(idx[:, 0], minlength=k) / N
        want = scipy.special.softmax(e / T)
        assert np.all(np.abs(share - want) <= 1.0 / N + 1e-12), f"T={T}: {share} vs {want}"
        # the stratified draws are monotone in u: indices never decrease
        assert np.all(np.diff(idx[:, 0]) >= 0)


def pin_sample_low_temperature_is_greedy(o):
    # a temperature far below every gap between a row's edges concentrates the draw on the
    # argmax: the sampled walk equals the (enumeration-pinned) greedy walk, predecessors included
    rng = np.random.default_rng(62)
    B, L, k = 3, 5, 6
    edges = rng.permutation(B * L * k * k).reshape(B, L, k, k).astype(np.float64)  # gaps >= 1
    edges[:, 0] = edges[:, 0, :1]
    cand = rng.integers(0, 1000, (B, L, k)).astype(np.int32)
    u = rng.uniform(0.02, 0.98, (B, L))
    path_g, idx_g, _, _ = o.walk(edges, cand)
    path_s, idx_s, _, _, _ = o.walk_ex(edges, cand, 0.01, u, 0.0)
    assert np.array_equal(idx_s, idx_g) and np.array_equal(path_s, path_g)
    path_0, idx_0, _, _, _ = o.walk_ex(edges, cand, 0.0, None, 0.0)   # T = 0: greedy itself
    assert np.array_equal(idx_0, idx_g)


def pin_sample_follows_predecessor(o):
    # position 1's row i puts (almost) all mass on index i: the draw there must repeat the index
    # drawn at position 0, whatever it was
    k, B = 4, 64
    e0 = np.zeros(k)
    edges = np.zeros((B, 2, k, k))
    edges[:, 0] = e0
    edges[:, 1] = np.where(np.eye(k, dtype=bool), 0.0, -60.0)
    cand = np.tile(np.arange(k, dtype=np.int32), (B, 2, 1))
    u = np.stack([(np.arange(B) + 0.5) / B, np.full(B, 0.5)], 1)
    _, idx, _, _, _ = o.walk_ex(edges, cand, 1.0, u, 0.0)
    assert np.array_equal(idx[:, 1], idx[:, 0])
    assert np.array_equal(np.bincount(idx[:, 0], minlength=k), np.full(k, B // k))


def pin_pmin_closed_form(o):
    # two candidates d apart: the greedy confidence is 1 / (1 + e^-d); the block ends before the
    # first position below p_min
    d = np.array([2.0, 1.0, 0.5, 3.0])
    L = len(d)
    edges = np.zeros((1, L, 2, 2))
    edges[0, :, :, 1] = d[:, None]
    cand = np.tile(np.array([7, 8], np.int32), (1, L, 1))
    conf_want = 1.0 / (1.0 + np.exp(-d))
    for p_min, want_len in [(0.0, 4), (0.6, 4), (0.7, 2), (0.8, 1), (0.9, 0), (1.0, 0)]:
        _, idx, dlen, conf, _ = o.walk_ex(edges, cand, 0.0, None, p_min)
        assert np.all(idx == 1)
        assert np.allclose(conf[0], conf_want, rtol=1e-14, atol=0)
        assert dlen[0] == want_len, f"p_min={p_min}: draft_len {dlen[0]} vs {want_len}"
    # a confidence exactly at p_min does not stop the block (strictly below stops it)
    edges = np.zeros((1, 3, 2, 2))
    _, _, dlen, conf, _ = o.walk_ex(edges, np.zeros((1, 3, 2), np.int32), 0.0, None, 0.5)
    assert np.all(conf == 0.5) and dlen[0] == 3
    # k = 1: the confidence is 1, so only p_min > 1 ends the block at once
    e1 = np.zeros((2, 3, 1, 1))
    c1 = np.zeros((2, 3, 1), np.int32)
    assert np.all(o.walk_ex(e1, c1, 0.0, None, 1.0)[2] == 3)
    assert np.all(o.walk_ex(e1, c1, 0.0, None, 1.5)[2] == 0)


def pin_sampled_confidence_and_margin(o):
    # row (0, ln 3): probabilities 1/4 and 3/4. u = 0.2 draws index 0 (running sums 1/4, 1), so
    # its confidence is 1/4 and the draw sits 0.05 of the total from the nearest boundary
    edges = np.zeros((1, 1, 2, 2))
    edges[0, 0, :, 1] = math.log(3.0)
    cand = np.array([[[5, 9]]], np.int32)
    _, idx, dlen, conf, cm = o.walk_ex(edges, cand, 1.0, np.array([[0.2]]), 0.3)
    assert idx[0, 0] == 0 and abs(conf[0, 0] - 0.25) < 1e-15 and abs(cm[0, 0] - 0.05) < 1e-15
    assert dlen[0] == 0   # 1/4 < 0.3
    _, idx, _, conf, cm = o.walk_ex(edges, cand, 1.0, np.array([[0.3]]), 0.0)
    assert idx[0, 0] == 1 and abs(conf[0, 0] - 0.75) < 1e-15 and abs(cm[0, 0] - 0.05) < 1e-15
    # at T = 2 the probabilities are 1 / (1 + sqrt 3) and sqrt 3 / (1 + sqrt 3)
    p0 = 1.0 / (1.0 + math.sqrt(3.0))
    _, idx, _, conf, _ = o.walk_ex(edges, cand, 2.0, np.array([[p0 - 1e-6]]), 0.0)
    assert idx[0, 0] == 0 and abs(conf[0, 0] - 0.25) < 1e-15   # confidence is not scaled by T
    _, idx, _, _, _ = o.walk_ex(edges, cand, 2.0, np.array([[p0 + 1e-6]]), 0.0)
    assert idx[0, 0] == 1


# ------------------------------------------------------ grouped dynamic depthwise convolution

def _conv_inputs(rng, nb, T, C, K, G, dtype=F32):
    x = rng.normal(0, 1, (nb, T, C)).astype(np.float32)
    base = rng.normal(0, 0.5, (K, C)).astype(np.float32)
    dyn = rng.normal(0, 0.2, (nb, T, K, C // G)).astype(np.float32)
    if dtype == BF16:
        cut = lambda a: (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        return bf16_bits(cut(x)), bf16_bits(cut(base)), bf16_bits(cut(dyn))
    return x, base, dyn


def pin_conv_static_is_numpy_convolve(o):
    # with the dynamic part zero, every channel of every block is a causal FIR filter with the
    # channel's static taps: numpy's full convolution, truncated to the block
    rng = np.random.default_rng(71)
    for nb, T, C, K, G, dt in [(3, 9, 32, 2, 16, F32), (2, 17, 48, 3, 16, BF16), (1, 5, 8, 4, 4, F32)]:
        x, base, dyn = _conv_inputs(rng, nb, T, C, K, G, dt)
        dyn = np.zeros_like(dyn)
        y = o.dynconv(x, base, dyn, G)
        xw, bw = widen(x), widen(base)
        for b in range(nb):
            for c in range(C):
                want = np.convolve(xw[b, :, c], bw[:, c])[:T]
                assert np.allclose(y[b, :, c], want, rtol=1e-13, atol=1e-13)


def pin_conv_impulse(o):
    # a single 1 at (b, t0, c0): tap j carries it to row t0 + j of channel c0 only, with the
    # coefficient of that output row: base[j][c0] + dyn[b][t0 + j][j][c0 / G]
    rng = np.random.default_rng(72)
    nb, T, C, K, G = 2, 8, 32, 3, 16
    _, base, dyn = _conv_inputs(rng, nb, T, C, K, G)
    b, t0, c0 = 1, 4, 21
    x = np.zeros((nb, T, C), np.float32)
    x[b, t0, c0] = 1.0
    y = o.dynconv(x, base, dyn, G)
    want = np.zeros((nb, T, C))
    for j in range(K):
        if t0 + j < T:
            want[b, t0 + j, c0] = float(base[j, c0]) + float(dyn[b, t0 + j, j, c0 // G])
    assert np.allclose(y, want, rtol=1e-15, atol=0), "impulse response"


def pin_conv_block_local_and_grouped(o):
    rng = np.random.default_rng(73)
    nb, T, C, K, G = 3, 6, 64, 2, 16
    x, base, dyn = _conv_inputs(rng, nb, T, C, K, G)
    y = o.dynconv(x, base, dyn, G)
    # changing one block's inputs changes no other block (zero padding, not the previous block)
    x2 = x.copy()
    x2[1] += 1.0
    y2 = o.dynconv(x2, base, dyn, G)
    assert np.array_equal(y2[[0, 2]], y[[0, 2]]) and not np.allclose(y2[1], y[1])
    # row 0 of a block sees only tap 0
    assert np.allclose(y[:, 0], (base[0] + np.repeat(dyn[:, 0, 0], G, axis=1)) * x[:, 0],
                       rtol=1e-6, atol=1e-7)
    # a correction of group g moves exactly the G channels of that group, by x of that tap
    d2 = dyn.copy()
    d2[2, 3, 1, 2] += 0.5
    y3 = o.dynconv(x, base, d2, G)
    diff = y3 - y
    want = np.zeros_like(diff)
    delta = float(d2[2, 3, 1, 2]) - float(dyn[2, 3, 1, 2])   # the stored (fp32) change
    want[2, 3, 2 * G:3 * G] = delta * x[2, 2, 2 * G:3 * G].astype(np.float64)
    assert np.allclose(diff, want, rtol=1e-9, atol=1e-12), "group broadcast"


# ---------------------------------------------------------------------- LM-head top-k

def pin_lmhead_matmul_then_sort(o):
    rng = np.random.default_rng(41)
    for R, H, V, k, bf in [(3, 24, 50, 5, False), (4, 64, 700, 16, True), (1, 8, 16, 16, True)]:
        h = rng.normal(0, 1, (R, H)).astype(np.float32)
        w = (rng.normal(0, 3, (V, H)) / math.sqrt(H)).astype(np.float32)
        if bf:
            h = (h.view(np.uint32) & 0xFFFF0000).view(np.float32)
            w = (w.view(np.uint32) & 0xFFFF0000).view(np.float32)
            ids, unary, lse, x = o.lmhead_topk(bf16_bits(h), bf16_bits(w), k, want_logits=True)
        else:
            ids, unary, lse, x = o.lmhead_topk(h, w, k, want_logits=True)
        want = h.astype(np.float64) @ w.astype(np.float64).T
        scale = np.abs(h.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
        assert np.all(np.abs(x - want) <= 1e-13 * scale + 1e-300), "logits are hidden . W_lm^T"
        for i in range(R):
            order = sort_order(want[i])
            assert np.array_equal(ids[i], order[:k])
            want_lse = scipy.special.logsumexp(want[i])
            assert abs(lse[i] - want_lse) <= 1e-12 * max(1.0, abs(want_lse))
            assert np.allclose(unary[i], want[i][order[:k]] - want_lse, rtol=0, atol=1e-12)


def pin_lmhead_onehot_weight(o):
    rng = np.random.default_rng(42)
    R, H, V, k = 5, 16, 40, 6
    h = rng.normal(0, 1, (R, H)).astype(np.float32)
    hv = rng.integers(0, H, V)
    c = rng.choice([-2.0, -0.5, 0.25, 1.0, 3.0], V).astype(np.float32)
    w = np.zeros((V, H), np.float32)
    w[np.arange(V), hv] = c
    ids, unary, lse, x = o.lmhead_topk(h, w, k, want_logits=True)
    want = c[None, :].astype(np.float64) * h[:, hv].astype(np.float64)
    assert np.array_equal(x, want), "vocabulary row v reads hidden column h(v) only"
    for i in range(R):
        assert np.array_equal(ids[i], sort_order(want[i])[:k])


def pin_lmhead_zero_hidden(o):
    rng = np.random.default_rng(43)
    V, k = 97, 9
    w = rng.normal(0, 1, (V, 32)).astype(np.float32)
    ids, unary, lse = o.lmhead_topk(np.zeros((2, 32), np.float32), w, k)
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (2, 1)))
    assert np.allclose(lse, math.log(V), rtol=0, atol=1e-13)
    assert np.allclose(unary, -math.log(V), rtol=0, atol=1e-13)


PINS = [
    pin_topk_full_sort, pin_topk_bruteforce_rank, pin_topk_boundary_ties, pin_topk_signed_zero,
    pin_topk_shift_invariance, pin_lse_normalises, pin_lse_scipy, pin_unary_softmax,
    pin_constant_row, pin_bf16_values, pin_gate_matmul, pin_gate_onehot_rows, pin_gate_zero,
    pin_lattice_identity_gate, pin_lattice_onehot_codes, pin_lattice_zero_codebooks,
    pin_lattice_linear_in_gate, pin_lattice_anchor_rows, pin_walk_bruteforce,
    pin_walk_score_and_margin, pin_walk_edge_tie, pin_reduces_to_argmax, pin_sample_frequencies,
    pin_sample_low_temperature_is_greedy, pin_sample_follows_predecessor, pin_pmin_closed_form,
    pin_sampled_confidence_and_margin, pin_conv_static_is_numpy_convolve, pin_conv_impulse,
    pin_conv_block_local_and_grouped, pin_lmhead_matmul_then_sort, pin_lmhead_onehot_weight,
    pin_lmhead_zero_hidden,
]
