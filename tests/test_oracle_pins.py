"""Pins of the CPU oracle against things other than itself (CPU only).

Each check below fixes part of the oracle by an independent route:
hand-computed worked examples (tests/golden/*.json, derivations inline),
exact-rational brute force on tiny inputs (fractions.Fraction, selection by
repeated extraction rather than sorting), closed forms, special cases that
reduce to textbook routines, and invariants the pages state.  The mutation
tests at the end plant plausible mistakes in the oracle (a dropped ReLU, a
wrong mask boundary, a reversed tie-break, softmax over the wrong axis, ...)
and require that some pin fails for each.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.indexer as OI
import synthetic as SY

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    """JSON value -> float, with '-inf' strings."""
    if isinstance(x, list):
        return [_f(v) for v in x]
    return float("-inf") if x == "-inf" else float(x)


# ---------------------------------------------------------------------------
# Golden (hand-computed) examples
# ---------------------------------------------------------------------------

def check_golden_indexer():
    g = _load("indexer_tiny.json")
    q = np.array(g["q"], dtype=np.float64)
    k = np.array(g["k"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    for case in g["cases"]:
        idx, vals = oracle.score_topk(q, k, w, case["compress_ratio"], case["topk"])
        assert idx.tolist() == case["idx"], (case, idx.tolist())
        np.testing.assert_array_equal(vals, np.array(_f(case["scores"])))


def check_golden_kpool():
    g = _load("kpool_tiny.json")
    r = oracle.kpool_compress(np.array(g["k_normed"], dtype=np.float64),
                              np.array(g["gate"], dtype=np.float64),
                              np.array(g["valid"], dtype=np.uint8),
                              np.array(g["ape"], dtype=np.float64), g["first_key"], g["KP"])
    assert r["pool_k_bits"].tolist() == g["pool_k_bits"]
    assert r["pool_k"].tolist() == g["pool_k"]
    assert r["pool_tok"].tolist() == g["pool_tok"]
    assert r["pool_valid"].tolist() == g["pool_valid"]


def check_golden_pooled():
    g = _load("pooled_tiny.json")
    q = np.array(g["q"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    pk = np.array(g["pool_k"], dtype=np.float64)
    pv = np.array(g["pool_valid"], dtype=np.uint8)
    sc = oracle.pooled_index_scores(q, w, pk, pv)
    np.testing.assert_array_equal(sc, np.array(_f(g["scores"])))
    for case in g["cases"]:
        sel = case["index_topk"] // g["KP"]
        ids, vals = oracle.topk_pools(sc, sel)
        assert ids.tolist() == case["pool_ids"]
        np.testing.assert_array_equal(vals, np.array(_f(case["pool_scores"])))
        tok = oracle.expand_selection(ids, g["first_key"], g["KP"])
        assert tok.tolist() == case["tokens"]


def test_golden_indexer():
    check_golden_indexer()


def test_golden_kpool():
    check_golden_kpool()


def test_golden_pooled():
    check_golden_pooled()


# ---------------------------------------------------------------------------
# Exact-rational brute force on tiny inputs
# ---------------------------------------------------------------------------

def _brute_visible(s, t, Skv, r):
    # compressed key s summarises tokens r*s .. r*s+r-1; visible once all are <= t
    return s < Skv and r * (s + 1) <= t + 1


def _brute_pick(scores, topk):
    """Repeatedly extract the best remaining key: highest score, then lowest index."""
    remaining = dict(scores)
    chosen = []
    while len(chosen) < topk and remaining:
        best = None
        for s in sorted(remaining):
            if best is None or remaining[s] > remaining[best]:
                best = s
        chosen.append(best)
        del remaining[best]
    return chosen


def brute_score_topk(q, k, w, r, topk):
    S, B, H, D = q.shape
    Skv = k.shape[0]
    F = lambda x: Fraction(float(x))
    idx = np.full((B, S, topk), -1, dtype=np.int64)
    vals = [[[None] * topk for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for t in range(S):
            scores = {}
            for s in range(Skv):
                if not _brute_visible(s, t, Skv, r):
                    continue
                tot = Fraction(0)
                for h in range(H):
                    dot = sum((F(q[t, b, h, d]) * F(k[s, b, d]) for d in range(D)), Fraction(0))
                    tot += F(w[t, b, h]) * max(dot, Fraction(0))
                scores[s] = tot
            chosen = _brute_pick(scores, topk)
            for i, s in enumerate(chosen):
                idx[b, t, i] = s
                vals[b][t][i] = scores[s]
    return idx, vals


# Short-mantissa value sets: many exact ties, every fp64 step of the oracle exact.
_QK_SET = np.array([-2, -1.5, -1, -0.5, -0.25, 0, 0, 0.25, 0.5, 1, 1.5, 2, 0.375, -0.125])
_W_SET = np.array([-1, -0.5, 0, 0.25, 0.5, 1, 2, -2])


def _tiny_case(rng, S, Skv, B, H, D, discrete=True):
    if discrete:
        q = rng.choice(_QK_SET, (S, B, H, D))
        k = rng.choice(_QK_SET, (Skv, B, D))
    else:  # random bf16 values
        q = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(rng.standard_normal((S, B, H, D)).astype(np.float32)))
        k = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(rng.standard_normal((Skv, B, D)).astype(np.float32)))
    w = rng.choice(_W_SET, (S, B, H))
    return q.astype(np.float64), k.astype(np.float64), w.astype(np.float64)


def check_bruteforce_score_topk(n_cases=40, seed=1):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        S = int(rng.integers(1, 11))
        Skv = int(rng.integers(1, 11))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        D = int(rng.integers(1, 5))
        r = int(rng.integers(1, 4))
        topk = int(rng.integers(1, 13))
        q, k, w = _tiny_case(rng, S, Skv, B, H, D, discrete=(c % 3 != 2))
        idx, vals = oracle.score_topk(q, k, w, r, topk)
        bidx, bvals = brute_score_topk(q, k, w, r, topk)
        assert np.array_equal(idx, bidx), (c, idx, bidx)
        for b in range(B):
            for t in range(S):
                for i in range(topk):
                    if bidx[b, t, i] < 0:
                        assert vals[b, t, i] == -math.inf
                    else:
                        assert Fraction(float(vals[b, t, i])) == bvals[b][t][i]


def test_bruteforce_score_topk():
    check_bruteforce_score_topk()


def _tiny_offsets(rng, n, total_max):
    lens = rng.integers(0, total_max + 1, size=n)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def check_bruteforce_packed(n_cases=12, seed=11):
    """Packed sequences against one global brute force: every packed row t of
    sequence i (local position t - cu_q[i]) scores the global keys
    cu_k[i] .. cu_k[i] + min(len_k, floor((t_local + 1) / r)) - 1 exactly,
    ranks them by (score desc, global key asc) and reports them minus
    cu_k[i]; no per-sequence sub-problem is formed.  Also the supplied-index
    form at the rows' own selection."""
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        nseq = int(rng.integers(1, 4))
        cu_q, cu_k = _tiny_offsets(rng, nseq, 5), _tiny_offsets(rng, nseq, 6)
        Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
        H, D, r = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
        topk = int(rng.integers(1, 6))
        q = rng.choice(_QK_SET, (Tq, H, D)).astype(np.float64)
        k = rng.choice(_QK_SET, (max(Tk, 1), D)).astype(np.float64)[:Tk]
        w = rng.choice(_W_SET, (Tq, H)).astype(np.float64)
        idx, vals = oracle.score_topk_packed(q, k, w, cu_q, cu_k, r, topk)
        for i in range(nseq):
            for t in range(int(cu_q[i]), int(cu_q[i + 1])):
                tl = t - int(cu_q[i])
                n = min(int(cu_k[i + 1] - cu_k[i]), (tl + 1) // r)
                keys = list(range(int(cu_k[i]), int(cu_k[i]) + n))
                ex = []
                for g in keys:
                    tot = Fraction(0)
                    for h in range(H):
                        d = sum(Fraction(float(q[t, h, e])) * Fraction(float(k[g, e])) for e in range(D))
                        tot += Fraction(float(w[t, h])) * max(d, Fraction(0))
                    ex.append((-tot, g))
                ex.sort()
                want = [g - int(cu_k[i]) for _, g in ex[:topk]] + [-1] * max(0, topk - len(ex))
                assert list(idx[t]) == want, (c, i, t, list(idx[t]), want)
                for j, (negv, _) in enumerate(ex[:topk]):
                    assert Fraction(float(vals[t, j])) == -negv
                assert all(v == -math.inf for v in vals[t, len(ex):])
        sidx, svals = oracle.score_topk_packed(q, k, w, cu_q, cu_k, r, topk, topk_indices=idx)
        assert np.array_equal(sidx, idx) and np.array_equal(svals, vals), c


def test_bruteforce_packed():
    check_bruteforce_packed()


def check_backward_packed_finite_differences(n_cases=3, seed=12):
    """Packed backward: every input coordinate's gradient equals the central
    difference of L = sum of g * score over the usable supplied entries,
    with the scores from the packed forward (its supplied-index form), so
    the sequence slicing of the backward is checked against the forward's.
    Dyadic inputs with no zero product on a usable entry: exact."""
    rng = np.random.default_rng(seed)
    eps = 2.0 ** -12
    for c in range(n_cases):
        while True:
            nseq = 3
            cu_q, cu_k = _tiny_offsets(rng, nseq, 3), _tiny_offsets(rng, nseq, 4)
            Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
            H, D, r, n = int(rng.integers(1, 3)), int(rng.integers(2, 4)), 1, 3
            q = rng.choice(_QK_SET, (Tq, H, D)).astype(np.float64)
            k = rng.choice(_QK_SET, (Tk, D)).astype(np.float64)
            w = rng.choice(_W_SET, (Tq, H)).astype(np.float64)
            sup = rng.integers(-1, 5, size=(Tq, n)).astype(np.int32)
            g = rng.choice(_G_SET, (Tq, n)).astype(np.float64)
            zero = False
            for i in range(nseq):
                for t in range(int(cu_q[i]), int(cu_q[i + 1])):
                    nt = min(int(cu_k[i + 1] - cu_k[i]), t - int(cu_q[i]) + 1)
                    for s in sup[t]:
                        if 0 <= s < nt and np.any(q[t] @ k[int(cu_k[i]) + s] == 0):
                            zero = True
            if Tq > 0 and Tk > 0 and not zero:
                break

        def loss():
            _, v = oracle.score_topk_packed(q, k, w, cu_q, cu_k, r, n, topk_indices=sup)
            ok = np.isfinite(v)
            return float(np.sum(np.where(ok, v, 0.0) * g))
        got = oracle.indexer_backward_packed(q, k, w, cu_q, cu_k, r, sup, g)
        for name, arr in (("grad_q", q), ("grad_k", k), ("grad_w", w)):
            fd = np.zeros(arr.shape)
            for pos in np.ndindex(*arr.shape):
                keep = arr[pos]
                arr[pos] = keep + eps
                hi = loss()
                arr[pos] = keep - eps
                lo = loss()
                arr[pos] = keep
                fd[pos] = (hi - lo) / (2 * eps)
            assert np.array_equal(got[name], fd), (c, name, np.argwhere(got[name] != fd)[:4])


def test_backward_packed_finite_differences():
    check_backward_packed_finite_differences()


def _brute_bf16(x: Fraction) -> Fraction:
    """Nearest bf16 value to an exact rational, ties to the even significand."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2): 8 significant bits -> step 2**-7
    scaled = a * 128
    lo = math.floor(scaled)
    frac = scaled - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * Fraction(lo, 128) * (Fraction(2) ** e)


def check_round_to_bf16(seed=2):
    rng = np.random.default_rng(seed)
    xs = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-3, 4, 300),
                         # exact midpoints between neighbouring bf16 values
                         [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 + 2.0 ** -7,
                          2.0 ** -8 * 257, 0.0, 1.0, -2.5]])
    vals, bits = oracle.round_to_bf16(xs)
    for x, v, b in zip(xs, vals, bits):
        exp = _brute_bf16(Fraction(float(x)))
        assert Fraction(float(v)) == exp, (x, v, exp)
        assert float(SY.bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0]) == float(exp)


def test_round_to_bf16_bruteforce():
    check_round_to_bf16()


def check_bruteforce_pooled(seed=3):
    """Pooled pipeline in exact rationals where the softmax is exact:
    uniform logits (weights exactly 1/KP for KP a power of two) and KP = 1."""
    rng = np.random.default_rng(seed)
    for KP in (1, 2, 4):
        N, D, H, Q = 23, 3, 2, 4
        first_key = int(rng.integers(0, 4))
        kn = rng.choice(_QK_SET, (N, D)).astype(np.float64)
        gate = np.full((N, D), 0.75)            # uniform logits per channel
        ape = np.zeros((KP, D))
        valid = (rng.random(N) < 0.85).astype(np.uint8)
        r = oracle.kpool_compress(kn, gate, valid, ape, first_key, KP)
        P = (N - first_key) // KP
        assert r["pool_k"].shape == (P, D)
        exact_pk = []
        for p in range(P):
            toks = [first_key + p * KP + j for j in range(KP)]
            row = []
            for c in range(D):
                mean = sum((Fraction(float(kn[t, c])) for t in toks), Fraction(0)) / KP
                row.append(_brute_bf16(mean))
            exact_pk.append(row)
            assert r["pool_valid"][p] == (1 if all(valid[t] for t in toks) else 0)
            assert r["pool_tok"][p] == toks[0]
        assert [[Fraction(float(v)) for v in row] for row in r["pool_k"]] == exact_pk
        # pooled scores + selection, brute force on the exact pool keys
        q = rng.choice(_QK_SET, (Q, H, D)).astype(np.float64)
        w = rng.choice(_W_SET, (Q, H)).astype(np.float64)
        sc = oracle.pooled_index_scores(q, w, r["pool_k"], r["pool_valid"])
        for sel in (1, 3, P + 2):
            ids, vals = oracle.topk_pools(sc, sel)
            for i in range(Q):
                scores = {}
                for p in range(P):
                    if not r["pool_valid"][p]:
                        continue
                    tot = Fraction(0)
                    for h in range(H):
                        dot = sum((Fraction(float(q[i, h, c])) * exact_pk[p][c] for c in range(D)),
                                  Fraction(0))
                        tot += Fraction(float(w[i, h])) * max(dot, Fraction(0))
                    scores[p] = tot
                chosen = _brute_pick(scores, sel)
                assert ids[i].tolist() == chosen + [-1] * (sel - len(chosen))
                for j, p in enumerate(chosen):
                    assert Fraction(float(vals[i, j])) == scores[p]


def test_bruteforce_pooled():
    check_bruteforce_pooled()


def check_bruteforce_pool_limits(n_cases=12, seed=31):
    """Per-row visible-pool bounds: each row selects, by exact rational
    arithmetic, only among valid pools p < its bound (bounds below 0 act as
    0, above P as P); the selection is the brute-force one, ties to the lower
    pool id, padding where too few pools remain."""
    rng = np.random.default_rng(seed)
    F = lambda x: Fraction(float(x))
    for c in range(n_cases):
        P, D, H, Q = int(rng.integers(1, 9)), int(rng.integers(1, 4)), int(rng.integers(1, 3)), 5
        pk = rng.choice(_QK_SET, (P, D)).astype(np.float64)
        pv = (rng.random(P) < 0.8).astype(np.uint8)
        q = rng.choice(_QK_SET, (Q, H, D)).astype(np.float64)
        w = rng.choice(_W_SET, (Q, H)).astype(np.float64)
        lim = rng.integers(-2, P + 3, size=Q)
        sc = oracle.pooled_index_scores(q, w, pk, pv, pool_limit=lim)
        for sel in (1, 2, P + 1):
            ids, vals = oracle.topk_pools(sc, sel)
            for i in range(Q):
                scores = {}
                for p_ in range(min(max(int(lim[i]), 0), P)):
                    if not pv[p_]:
                        continue
                    tot = Fraction(0)
                    for h in range(H):
                        dot = sum((F(q[i, h, d]) * F(pk[p_, d]) for d in range(D)), Fraction(0))
                        tot += F(w[i, h]) * max(dot, Fraction(0))
                    scores[p_] = tot
                chosen = _brute_pick(scores, sel)
                assert ids[i].tolist() == chosen + [-1] * (sel - len(chosen)), (c, i)
                for j, p_ in enumerate(chosen):
                    assert F(vals[i, j]) == scores[p_]


def check_pool_limit_reduces_to_unbounded(seed=32):
    """A bound of P (or more) for every row is the call without bounds."""
    rng = np.random.default_rng(seed)
    P, D, H, Q = 40, 8, 4, 6
    pk = rng.standard_normal((P, D))
    pv = (rng.random(P) < 0.9).astype(np.uint8)
    q, w = rng.standard_normal((Q, H, D)), rng.standard_normal((Q, H))
    ref = oracle.pooled_index_scores(q, w, pk, pv)
    for lim in (np.full(Q, P), np.full(Q, P + 7)):
        assert np.array_equal(oracle.pooled_index_scores(q, w, pk, pv, pool_limit=lim), ref)
    none = oracle.pooled_index_scores(q, w, pk, pv, pool_limit=np.zeros(Q, np.int64))
    assert np.all(np.isneginf(none))


def test_bruteforce_pool_limits():
    check_bruteforce_pool_limits()


def test_pool_limit_reduces_to_unbounded():
    check_pool_limit_reduces_to_unbounded()


# ---------------------------------------------------------------------------
# Special cases, closed forms, invariants
# ---------------------------------------------------------------------------

def test_single_head_unit_weight_is_relu_qk_topk():
    """H = 1, w = 1: I = ReLU(q . k); the causal top-k is a stable argsort of
    the masked row of ReLU(Q K^T) (numpy matmul + stable argsort)."""
    rng = np.random.default_rng(4)
    S, D = 40, 8
    q = rng.standard_normal((S, 1, 1, D))
    k = rng.standard_normal((S, 1, D))
    w = np.ones((S, 1, 1))
    idx, vals = oracle.score_topk(q, k, w, 1, 10)
    M = np.maximum(q[:, 0, 0, :] @ k[:, 0, :].T, 0.0)
    for t in range(S):
        row = M[t, : t + 1]
        order = np.argsort(-row, kind="stable")[:10]
        exp = np.full(10, -1)
        exp[: len(order)] = order
        assert idx[0, t].tolist() == exp.tolist()


def test_positive_homogeneity_in_keys():
    """Scaling a key by 4 (exact) scales every head dot product, hence the
    score, by exactly 4 (ReLU and the weighted sum are positively homogeneous)."""
    rng = np.random.default_rng(5)
    H, D, n = 8, 16, 30
    q = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(rng.standard_normal((H, D)).astype(np.float32)))
    k = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(rng.standard_normal((n, D)).astype(np.float32)))
    w = np.array([0.5, -0.25, 1, 2, -1, 0.125, 0.75, -0.5])
    s1 = oracle.head_scores(q, k, w)
    s4 = oracle.head_scores(q, 4.0 * k, w)
    np.testing.assert_array_equal(s4, 4.0 * s1)


def test_mask_closed_forms():
    # r = 4, S = 4M queries, Skv >= M: sum_t n_t = 2M^2 - M
    for M in (1, 2, 5, 1024, 4096):
        tot = sum(oracle.visible_keys(t, 10 ** 9, 4) for t in range(4 * M))
        assert tot == 2 * M * M - M
    # the c4 workload: 2M^2 - M = 33,550,336 visible pairs per batch at S = 16384
    assert sum(oracle.visible_keys(t, 4096, 4) for t in range(16384)) == 33550336
    # r = 1 with Skv >= S is the plain causal mask
    assert [oracle.visible_keys(t, 100, 1) for t in range(5)] == [1, 2, 3, 4, 5]
    # rows t < r - 1 see nothing
    assert [oracle.visible_keys(t, 100, 4) for t in range(5)] == [0, 0, 0, 1, 1]
    # capped at Skv
    assert oracle.visible_keys(10 ** 6, 4096, 1) == 4096


def check_invariants(seed=6):
    rng = np.random.default_rng(seed)
    for (S, Skv, r, topk) in ((97, 97, 1, 7), (120, 40, 3, 16), (50, 50, 1, 64), (33, 12, 2, 5)):
        q = rng.standard_normal((S, 2, 3, 5))
        k = rng.standard_normal((Skv, 2, 5))
        w = rng.standard_normal((S, 2, 3))
        idx, vals = oracle.score_topk(q, k, w, r, topk)
        for b in range(2):
            for t in range(S):
                n_t = oracle.visible_keys(t, Skv, r)
                row = idx[b, t]
                sel = row[row >= 0]
                assert np.all(sel < n_t)
                assert len(set(sel.tolist())) == len(sel)
                assert int(np.sum(row < 0)) == max(0, topk - n_t)
                assert np.all(row[len(sel):] == -1)        # padding only at the tail
                v = vals[b, t][: len(sel)]
                assert np.all(v[:-1] >= v[1:])            # non-increasing
                assert np.all(np.isneginf(vals[b, t][len(sel):]))
                # nothing unselected beats the last selected key
                if len(sel) < n_t and len(sel) > 0:
                    full = oracle.head_scores(q[t, b], k[:n_t, b], w[t, b])
                    rest = np.setdiff1d(np.arange(n_t), sel)
                    assert np.all(full[rest] <= v[-1])


def test_invariants():
    check_invariants()


def test_signed_zero_ties_resolve_by_index():
    # w < 0 times ReLU(negative) = -0.0; all-negative heads give +-0 scores
    q = np.array([[[[-1.0]]]])            # one query
    k = np.array([[[1.0]], [[1.0]], [[-1.0]]])
    w = np.array([[[-1.0]]])
    # t = 0 sees one key; use a later position by passing rows
    idx, vals = oracle.score_topk(q, k, w, 1, 3, rows=[2])
    # scores: s0: -1*ReLU(-1) = -0.0, s1: -0.0, s2: -1*ReLU(1) = -1
    assert idx[0, 0].tolist() == [0, 1, 2]
    assert vals[0, 0, 2] == -1.0


def check_kpool_invariants(seed=7):
    rng = np.random.default_rng(seed)
    N, D = 45, 6
    kn = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32)))
    gate = rng.standard_normal((N, D)).astype(np.float32)
    valid = (rng.random(N) < 0.8).astype(np.uint8)
    for KP in (1, 2, 3, 4, 8):
        ape = rng.standard_normal((KP, D)).astype(np.float32)
        for fk in (0, 3):
            r = oracle.kpool_compress(kn, gate, valid, ape, fk, KP)
            P = r["pool_k"].shape[0]
            assert P == max(0, N - fk) // KP
            for p in range(P):
                toks = fk + p * KP + np.arange(KP)
                # the pooled key lies within the slots' per-channel range
                assert np.all(r["pool_k_f64"][p] >= kn[toks].min(axis=0) - 1e-12)
                assert np.all(r["pool_k_f64"][p] <= kn[toks].max(axis=0) + 1e-12)
                assert r["pool_valid"][p] == int(all(valid[toks]))
                assert r["pool_tok"][p] == toks[0]
            if KP == 1:  # one slot: softmax weight 1, pool key == the token key
                assert np.array_equal(r["pool_k"], kn[fk:fk + P].astype(np.float64))
            # adding a constant to every logit of a channel changes nothing
            r2 = oracle.kpool_compress(kn, gate.astype(np.float64) + 1.0, valid, ape, fk, KP)
            np.testing.assert_allclose(r2["pool_k_f64"], r["pool_k_f64"], rtol=1e-14, atol=1e-14)
            # one dominant slot (+100 logit) copies that slot's key
            g3 = gate.astype(np.float64).copy()
            dom = KP - 1
            for p in range(P):
                g3[fk + p * KP + dom] += 100.0
            r3 = oracle.kpool_compress(kn, g3, valid, ape, fk, KP)
            if P:
                exp = kn[fk + dom: fk + P * KP: KP].astype(np.float64)
                assert np.array_equal(r3["pool_k"], exp)
    # permuting the slots of every pool together with the ape rows changes nothing
    KP = 4
    ape = rng.standard_normal((KP, D)).astype(np.float32)
    perm = np.array([2, 0, 3, 1])
    P = N // KP
    src = np.concatenate([p * KP + perm for p in range(P)] + [np.arange(P * KP, N)])
    r = oracle.kpool_compress(kn, gate, valid, ape, 0, KP)
    rp = oracle.kpool_compress(kn[src], gate[src], valid[src], ape[perm], 0, KP)
    np.testing.assert_allclose(rp["pool_k_f64"], r["pool_k_f64"], rtol=1e-14, atol=1e-14)
    assert np.array_equal(rp["pool_valid"], r["pool_valid"])


def test_kpool_invariants():
    check_kpool_invariants()


def test_kpool_degenerate_sizes():
    kn = np.ones((5, 2))
    g = np.zeros((5, 2))
    v = np.ones(5, dtype=np.uint8)
    a = np.zeros((4, 2))
    assert oracle.kpool_compress(kn, g, v, a, 5, 4)["pool_k"].shape == (0, 2)   # N == first_key
    assert oracle.kpool_compress(kn, g, v, a, 7, 4)["pool_k"].shape == (0, 2)   # N < first_key
    assert oracle.kpool_compress(kn, g, v, a, 2, 4)["pool_k"].shape == (0, 2)   # only a partial pool
    assert oracle.kpool_compress(kn, g, v, a, 1, 4)["pool_k"].shape == (1, 2)


def check_expand(seed=8):
    for KP in (1, 3, 4, 8):
        for fk in (0, 17):
            ids = SY.random_pool_ids(seed + KP, 5, 7, 50, missing_frac=0.3)
            tok = oracle.expand_selection(ids, fk, KP)
            assert tok.shape == (5, 7 * KP)
            for qi in range(5):
                for i in range(7):
                    seg = tok[qi, i * KP:(i + 1) * KP]
                    if ids[qi, i] == -1:
                        assert np.all(seg == -1)
                    else:
                        assert seg.tolist() == list(range(fk + KP * int(ids[qi, i]),
                                                          fk + KP * int(ids[qi, i]) + KP))
            # -1 exactly at the missing pools' slots, every slot written
            assert int(np.sum(tok == -1)) == KP * int(np.sum(ids == -1))


def test_expand():
    check_expand()


def test_topk_pools_fewer_valid_than_select():
    sc = np.array([[1.0, -np.inf, 3.0, -np.inf], [-np.inf] * 4])
    ids, vals = oracle.topk_pools(sc, 3)
    assert ids.tolist() == [[2, 0, -1], [-1, -1, -1]]
    assert np.isneginf(vals[1]).all()


def test_pooled_matches_unpooled_when_kp1():
    """KP = 1, ape = 0, all valid: pool keys are the token keys, so the pooled
    scores equal the unpooled scores of a query that sees every key."""
    rng = np.random.default_rng(9)
    N, D, H, Q = 64, 8, 4, 3
    kn = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(rng.standard_normal((N, D)).astype(np.float32)))
    r = oracle.kpool_compress(kn, rng.standard_normal((N, D)), np.ones(N, np.uint8), np.zeros((1, D)), 0, 1)
    q = rng.standard_normal((Q, H, D))
    w = rng.standard_normal((Q, H))
    sc = oracle.pooled_index_scores(q, w, r["pool_k"], r["pool_valid"])
    ids, _ = oracle.topk_pools(sc, 9)
    qs = q[:, None, :, :]
    ws = w[:, None, :]
    idx, _ = oracle.score_topk(np.repeat(qs, 1, axis=0), kn[:, None, :], ws, 1, 9,
                               rows=[N - 1 + i for i in range(Q)])
    assert np.array_equal(ids, idx[0])


# ---------------------------------------------------------------------------
# Scores at supplied indices
# ---------------------------------------------------------------------------

def check_bruteforce_scores_at_indices(n_cases=30, seed=5):
    """Exact rational scores at random supplied indices, including -1,
    out-of-range, masked (s >= n_t) and repeated entries."""
    rng = np.random.default_rng(seed)
    F = lambda x: Fraction(float(x))
    for c in range(n_cases):
        S, Skv = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        B, H, D = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 5))
        r, n = int(rng.integers(1, 4)), int(rng.integers(1, 10))
        q, k, w = _tiny_case(rng, S, Skv, B, H, D, discrete=(c % 3 != 2))
        sup = rng.integers(-2, Skv + 3, size=(B, S, n))
        idx, vals = oracle.scores_at_indices(q, k, w, r, sup)
        for b in range(B):
            for t in range(S):
                for j in range(n):
                    s = int(sup[b, t, j])
                    if s < 0 or not _brute_visible(s, t, Skv, r):
                        assert idx[b, t, j] == -1 and vals[b, t, j] == -math.inf, (c, b, t, j)
                        continue
                    tot = Fraction(0)
                    for h in range(H):
                        dot = sum((F(q[t, b, h, d]) * F(k[s, b, d]) for d in range(D)), Fraction(0))
                        tot += F(w[t, b, h]) * max(dot, Fraction(0))
                    assert idx[b, t, j] == s and Fraction(float(vals[b, t, j])) == tot, (c, b, t, j)


def check_scores_at_own_topk():
    """Fed the indices score_topk selected, the gather returns exactly the
    scores score_topk reported, padding included."""
    rng = np.random.default_rng(9)
    q, k, w = _tiny_case(rng, 40, 30, 2, 3, 8, discrete=False)
    for r, topk in ((1, 7), (3, 12), (2, 40)):
        idx, vals = oracle.score_topk(q, k, w, r, topk)
        gi, gv = oracle.scores_at_indices(q, k, w, r, idx)
        assert np.array_equal(gi, idx) and np.array_equal(gv, vals)


def test_bruteforce_scores_at_indices():
    check_bruteforce_scores_at_indices()


def test_scores_at_own_topk():
    check_scores_at_own_topk()


# ---------------------------------------------------------------------------
# k_norm (LayerNorm with a bias)
# ---------------------------------------------------------------------------

def check_k_norm_hand_example():
    """x = [1, 2, 3, 4]: mean 2.5, biased variance (2.25+0.25+0.25+2.25)/4 =
    1.25; with eps = 0.25 the divisor is sqrt(1.5), and d/sqrt(1.5) for
    d = -1.5, -0.5, 0.5, 1.5 is -sqrt(1.5), -sqrt(1/6), sqrt(1/6), sqrt(1.5).
    gamma = [2, 1, 1, 0.5], beta = [0, 1, -1, 0.25] give
    [-2 sqrt(1.5), 1 - sqrt(1/6), sqrt(1/6) - 1, 0.5 sqrt(1.5) + 0.25]."""
    r = oracle.k_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([2.0, 1.0, 1.0, 0.5]),
                      np.array([0.0, 1.0, -1.0, 0.25]), 0.25)
    expect = [-2.449489742783178, 0.5917517095361369, -0.5917517095361369, 0.8623724356957945]
    assert np.allclose(r["k_normed_f64"][0], expect, rtol=0, atol=1e-14), r["k_normed_f64"]
    # bf16 of those: 8 significant bits
    assert np.array_equal(r["k_normed"][0], [-2.453125, 0.58984375, -0.58984375, 0.86328125])


def check_k_norm_properties():
    rng = np.random.default_rng(17)
    x = SY.bf16_bits_to_f32(SY.f32_to_bf16_bits(
        (rng.standard_normal((50, 128)) * 3 + rng.standard_normal((50, 1)) * 5).astype(np.float32)))
    x = x.astype(np.float64)
    eps = 1e-5
    plain = oracle.k_norm(x, np.ones(128), np.zeros(128), eps)["k_normed_f64"]
    # zero mean; variance var / (var + eps)
    var = x.var(axis=1)
    assert np.all(np.abs(plain.mean(axis=1)) < 1e-12)
    assert np.allclose(plain.var(axis=1), var / (var + eps), rtol=1e-12, atol=0)
    # a constant shift of a row changes nothing; with eps = 0 neither does a
    # positive scale
    shifted = oracle.k_norm(x + 7.25, np.ones(128), np.zeros(128), eps)["k_normed_f64"]
    assert np.allclose(shifted, plain, rtol=0, atol=1e-11)
    a0 = oracle.k_norm(x, np.ones(128), np.zeros(128), 0.0)["k_normed_f64"]
    a3 = oracle.k_norm(3.0 * x, np.ones(128), np.zeros(128), 0.0)["k_normed_f64"]
    assert np.allclose(a0, a3, rtol=0, atol=1e-12)
    # the library LayerNorm (fp64, biased variance, eps inside the root,
    # elementwise affine) agrees before rounding
    import torch
    g = rng.standard_normal(128)
    b = rng.standard_normal(128)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps).numpy()
    got = oracle.k_norm(x, g, b, eps)["k_normed_f64"]
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_k_norm_hand_example():
    check_k_norm_hand_example()


def test_k_norm_properties():
    check_k_norm_properties()


# ---------------------------------------------------------------------------
# Backward (gradients of the selected scores)
# ---------------------------------------------------------------------------

_G_SET = np.array([-2.0, -1.0, -0.5, 0.25, 0.5, 1.0, 1.5, 3.0])


def _selected_sum(q, k, w, r, sup, g):
    """sum over usable entries of g * (score at the entry), in fp64."""
    idx, vals = oracle.scores_at_indices(q, k, w, r, sup)
    ok = idx >= 0
    return float(np.sum(g[ok] * vals[ok]))


def _backward_case(rng, S, Skv, B, H, D, n):
    """Short-mantissa inputs where no usable (entry, head) dot product is 0,
    so the score is differentiable at the point (resampled until so)."""
    while True:
        q, k, w = _tiny_case(rng, S, Skv, B, H, D)
        r = int(rng.integers(1, 3))
        sup = rng.integers(-1, Skv + 1, size=(B, S, n))
        sup[:, :, 0] = rng.integers(0, Skv, size=(B, S))   # repeated entries are likely too
        g = rng.choice(_G_SET, (B, S, n))
        d = np.einsum("tbhd,sbd->btsh", q, k)
        zero = False
        for b in range(B):
            for t in range(S):
                for s in sup[b, t]:
                    if 0 <= s < oracle.visible_keys(t, Skv, r) and np.any(d[b, t, s] == 0):
                        zero = True
        if not zero:
            return q, k, w, r, sup, g


def check_backward_finite_differences(n_cases=6, seed=21):
    """Every input coordinate's gradient equals the central difference of
    the forward selected-score sum, exactly: the score is piecewise linear,
    the step 2^-12 crosses no kink (dot products are multiples of 2^-6 and
    move by at most 2^-11), and all fp64 steps are exact on these values."""
    rng = np.random.default_rng(seed)
    eps = 2.0 ** -12
    for c in range(n_cases):
        S, Skv, B, H, D, n = 5, 5, 2, int(rng.integers(1, 4)), int(rng.integers(2, 5)), 3
        q, k, w, r, sup, g = _backward_case(rng, S, Skv, B, H, D, n)
        got = oracle.indexer_backward(q, k, w, r, sup, g)
        for name, arr in (("grad_q", q), ("grad_k", k), ("grad_w", w)):
            fd = np.zeros(arr.shape)
            for pos in np.ndindex(*arr.shape):
                keep = arr[pos]
                arr[pos] = keep + eps
                hi = _selected_sum(q, k, w, r, sup, g)
                arr[pos] = keep - eps
                lo = _selected_sum(q, k, w, r, sup, g)
                arr[pos] = keep
                fd[pos] = (hi - lo) / (2 * eps)
            assert np.array_equal(got[name], fd), (c, name, np.argwhere(got[name] != fd)[:4])


def check_backward_euler(seed=22):
    """The score is positively homogeneous of degree 1 in w, in a query row's
    q and in each key, so by Euler's theorem sum(w * dL/dw) = sum(q * dL/dq)
    = sum(k * dL/dk) = L for L = sum of g * score over usable entries."""
    rng = np.random.default_rng(seed)
    for discrete in (True, False):
        q, k, w = _tiny_case(rng, 12, 10, 2, 3, 8, discrete=discrete)
        sup = rng.integers(-1, 11, size=(2, 12, 6))
        g = rng.standard_normal((2, 12, 6))
        L = _selected_sum(q, k, w, 2, sup, g)
        got = oracle.indexer_backward(q, k, w, 2, sup, g)
        for name, arr in (("grad_w", w), ("grad_q", q), ("grad_k", k)):
            assert math.isclose(float(np.sum(arr * got[name])), L, rel_tol=1e-12, abs_tol=1e-12), name


def check_backward_dense_form(seed=23):
    """Dense restatement with library matrix products: with G[t, s] the sum
    of g over row t's usable entries naming s, and per head h D_h = Q_h K^T,
    M_h = [D_h > 0]:  dQ_h = (w_h * G * M_h) K,  dK = sum_h (w_h * G * M_h)^T Q_h,
    dw_h = rowsum(G * ReLU(D_h))."""
    rng = np.random.default_rng(seed)
    S, Skv, H, D, n, r = 14, 11, 3, 6, 5, 2
    q, k, w = _tiny_case(rng, S, Skv, 1, H, D, discrete=False)
    sup = rng.integers(-1, Skv + 1, size=(1, S, n))
    g = rng.standard_normal((1, S, n))
    Gm = np.zeros((S, Skv))
    for t in range(S):
        for j in range(n):
            s = int(sup[0, t, j])
            if 0 <= s < oracle.visible_keys(t, Skv, r):
                Gm[t, s] += g[0, t, j]
    Q, K, W = q[:, 0], k[:, 0], w[:, 0]
    dK = np.zeros((Skv, D))
    got = oracle.indexer_backward(q, k, w, r, sup, g)
    for h in range(H):
        Dh = Q[:, h] @ K.T
        P = W[:, h:h + 1] * Gm * (Dh > 0)
        assert np.allclose(got["grad_q"][:, 0, h], P @ K, rtol=1e-12, atol=1e-12), h
        assert np.allclose(got["grad_w"][:, 0, h], (Gm * np.maximum(Dh, 0)).sum(axis=1),
                           rtol=1e-12, atol=1e-12), h
        dK += P.T @ Q[:, h]
    assert np.allclose(got["grad_k"][:, 0], dK, rtol=1e-12, atol=1e-12)


def check_backward_gate_at_zero():
    """A head whose dot product is exactly 0 passes no gradient to q or k
    (ReLU's derivative read as 0 there) and adds ReLU(0) = 0 to dL/dw."""
    q = np.zeros((1, 1, 2, 2))
    q[0, 0, 0] = [1.0, -1.0]          # head 0: q . k = 0
    q[0, 0, 1] = [1.0, 1.0]           # head 1: q . k = 2
    k = np.array([[[1.0, 1.0]]])
    w = np.array([[[3.0, 0.5]]])
    got = oracle.indexer_backward(q, k, w, 1, np.array([[[0]]]), np.array([[[2.0]]]))
    assert np.array_equal(got["grad_q"][0, 0], [[0.0, 0.0], [1.0, 1.0]])
    assert np.array_equal(got["grad_k"][0, 0], [1.0, 1.0])
    assert np.array_equal(got["grad_w"][0, 0], [0.0, 4.0])


def check_backward_bounds_consistent(seed=24):
    """abs_* bound |grad_*| and count_k counts the usable entries per key."""
    rng = np.random.default_rng(seed)
    q, k, w = _tiny_case(rng, 9, 7, 2, 3, 5, discrete=False)
    sup = rng.integers(-1, 8, size=(2, 9, 4))
    g = rng.standard_normal((2, 9, 4))
    got = oracle.indexer_backward(q, k, w, 1, sup, g, with_bounds=True)
    for x in ("q", "k"):
        assert np.all(np.abs(got["grad_" + x]) <= got["abs_" + x] * (1 + 1e-12))
        assert np.all(got["band_" + x] >= 0)
    assert np.all(np.abs(got["grad_w"]) <= got["abs_w"] * (1 + 1e-12))
    cnt = np.zeros((7, 2), dtype=np.int64)
    for b in range(2):
        for t in range(9):
            for s in sup[b, t]:
                if 0 <= s < oracle.visible_keys(t, 7, 1):
                    cnt[s, b] += 1
    assert np.array_equal(got["count_k"], cnt)


def test_backward_finite_differences():
    check_backward_finite_differences()


def test_backward_euler():
    check_backward_euler()


def test_backward_dense_form():
    check_backward_dense_form()


def test_backward_gate_at_zero():
    check_backward_gate_at_zero()


def test_backward_bounds_consistent():
    check_backward_bounds_consistent()


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

ALL_CHECKS = [check_golden_indexer, check_golden_kpool, check_golden_pooled,
              lambda: check_bruteforce_score_topk(12), check_round_to_bf16,
              check_bruteforce_pooled, check_invariants, check_kpool_invariants, check_expand,
              lambda: check_bruteforce_scores_at_indices(10), check_scores_at_own_topk,
              check_k_norm_hand_example, check_k_norm_properties,
              lambda: check_backward_finite_differences(2), check_backward_euler,
              check_backward_dense_form, check_backward_gate_at_zero,
              lambda: check_bruteforce_packed(6), lambda: check_backward_packed_finite_differences(1),
              check_bruteforce_pool_limits, check_pool_limit_reduces_to_unbounded]


def _some_check_fails():
    for chk in ALL_CHECKS:
        try:
            chk()
        except Exception:  # a failed assertion, or an error the mistake provokes
            return True
    return False


MUTANTS = {
    "relu dropped": ("_relu", lambda x: x),
    "relu after weighting": ("_weighted_head_sum",
                             lambda w, ph: np.maximum((w[:, None] * ph).sum(axis=0), 0.0)),
    "weights ignored": ("_weighted_head_sum", lambda w, ph: ph.sum(axis=0)),
    "mask s <= floor((t+1)/r)": ("visible_keys", lambda t, Skv, r: min(Skv, (t + 1) // r + 1)),
    "mask ignores ratio": ("visible_keys", lambda t, Skv, r: min(Skv, t + 1)),
    "mask uses t/r": ("visible_keys", lambda t, Skv, r: min(Skv, t // r)),
    "ties to higher index": ("rank_desc",
                             lambda s: np.lexsort((-np.arange(len(s)), -np.asarray(s, dtype=np.float64)))),
    "ascending order": ("rank_desc",
                        lambda s: np.lexsort((np.arange(len(s)), np.asarray(s, dtype=np.float64)))),
    "keys reversed": ("_dot_products", lambda q, k: q @ k[::-1].T),
    "gather admits s == n_t": ("_usable_keys", lambda s, n: (s >= 0) & (s <= n)),
    "layernorm unbiased variance": ("_row_moments", lambda x: (
        x.mean(axis=1, keepdims=True), x.var(axis=1, ddof=1, keepdims=True))),
    "layernorm eps outside the root": ("_inv_std", lambda var, eps: 1.0 / np.sqrt(var) + eps),
    "layernorm without centring": ("_row_moments", lambda x: (
        np.zeros((x.shape[0], 1)), x.var(axis=1, keepdims=True))),
    "gather admits masked keys": ("_usable_keys", lambda s, n: s >= 0),
    "softmax over channels": ("_slot_softmax",
                              lambda lg: np.exp(lg - lg.max(axis=1, keepdims=True)) /
                              np.exp(lg - lg.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)),
    "plain mean instead of softmax": ("_slot_softmax", lambda lg: np.full(lg.shape, 1.0 / lg.shape[0])),
    "partial trailing pool kept": ("pool_count", lambda N, fk, kp: max(0, -(-(N - fk) // kp))),
    "pooling ignores first_key": ("pool_count", lambda N, fk, kp: max(0, N // kp)),
    "backward gate is 1 at 0": ("_relu_gate", lambda d: (d >= 0).astype(np.float64)),
    "backward gate dropped": ("_relu_gate", lambda d: np.ones_like(d)),
    "backward gate inverted": ("_relu_gate", lambda d: (d < 0).astype(np.float64)),
    "backward ignores head weights": ("_gate_coef", lambda g, wp, on: g[:, None] * on),
    "backward drops the incoming gradient": ("_gate_coef", lambda g, wp, on: wp * on),
    "backward keys from the wrong batch": ("_pair_dots",
                                           lambda qp, kp: np.einsum("phd,pd->ph", qp, kp[::-1])),
    "packed keys from the batch start": ("_sequence_spans", lambda cq, ck: [
        (int(cq[i]), int(cq[i + 1]), 0, int(ck[i + 1] - ck[i])) for i in range(len(cq) - 1)]),
    "packed rows see the keys before them": ("_sequence_spans", lambda cq, ck: [
        (int(cq[i]), int(cq[i + 1]), 0, int(ck[i + 1])) for i in range(len(cq) - 1)]),
    "pool bound admits p == limit": ("visible_pools", lambda P, lim: (
        np.ones(P, dtype=bool) if lim is None else np.arange(P) <= min(max(int(lim), 0), P))),
    "pool bound ignored": ("visible_pools", lambda P, lim: np.ones(P, dtype=bool)),
    "negative pool bound wraps": ("visible_pools", lambda P, lim: (
        np.ones(P, dtype=bool) if lim is None else np.arange(P) < (int(lim) % (P + 1)))),
    "round toward zero": ("round_to_bf16", lambda x: (
        np.ldexp(np.trunc(np.ldexp(np.frexp(x)[0], 8)), np.frexp(x)[1] - 8),
        (np.ldexp(np.trunc(np.ldexp(np.frexp(x)[0], 8)), np.frexp(x)[1] - 8)
         .astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OI, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    assert _some_check_fails(), f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_all_checks():
    assert not _some_check_fails()
