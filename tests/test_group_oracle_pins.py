"""Pins of the grouped (approximate) indexer's CPU oracle
(oracle/csa_group_oracle.c), the query-group shared scan reading of the
PIVOT news item (themodelwire): groups of g consecutive positions pool
their queries, one scan of the keys the first member sees keeps C
candidates, and each member re-ranks them, plus its own extra keys, with
its exact scores.

Pinned by things other than the oracle itself:
  * exact rational brute force of the same reading in Python, with the
    pooled query rounded to bfloat16 by torch's cast (a library rounding);
  * reductions to the exact oracle: a candidate count covering every
    visible key, and groups of one position, give csa_oracle_rows' result;
  * invariants: set recall against the exact result never decreases with
    C, every returned key is visible and scored with the member's own
    exact score.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _case(rng, S, T, H, D, lo=-3, hi=3, wmax=3):
    q = rng.integers(lo, hi + 1, (S, H, D)).astype(np.float32)
    k = rng.integers(lo, hi + 1, (T, D)).astype(np.float32)
    w = rng.integers(0, wmax + 1, (S, H)).astype(np.float32)
    return _bf16_bits(q), w, _bf16_bits(k)


def _brute(qb, w, kb, rows, m, topk, g, C, row_offset=0):
    """The grouped reading with exact rationals; the pooled query's
    binary32 mean is formed with numpy float32 in member order and rounded
    to bfloat16 by torch's cast."""
    S, H, D = qb.shape
    T = kb.shape[0]
    qv = _bf16_value(qb)
    kf = [[Fraction(float(v)) for v in row] for row in _bf16_value(kb)]

    def nvis(t):
        return min(T, (t + 1) // m)

    def score(qrow, wrow, s):
        tot = Fraction(0)
        for j in range(H):
            dot = sum(Fraction(float(qrow[j][x])) * kf[s][x] for x in range(D))
            if dot > 0:
                tot += Fraction(float(wrow[j])) * dot
        return tot

    out_i, out_s = [], []
    for i in rows:
        i0 = (i // g) * g
        mem = range(i0, min(S, i0 + g))
        acc = np.zeros((H, D), np.float32)
        accw = np.zeros(H, np.float32)
        for u in mem:
            acc = (acc + qv[u].astype(np.float32)).astype(np.float32)
            accw = (accw + w[u]).astype(np.float32)
        n = np.float32(len(mem))
        pq = _bf16_value(_bf16_bits((acc / n).astype(np.float32)))
        pw = (accw / n).astype(np.float32)
        n0 = nvis(row_offset + i0)
        shared = sorted(range(n0), key=lambda s: (-score(pq, pw, s), s))[:C]
        keys = list(shared) + list(range(n0, nvis(row_offset + i)))
        ranked = sorted(keys, key=lambda s: (-score(qv[i], w[i], s), s))[:topk]
        sc = [float(score(qv[i], w[i], s)) for s in ranked]
        out_i.append(ranked + [-1] * (topk - len(ranked)))
        out_s.append(sc + [-np.inf] * (topk - len(ranked)))
    return np.array(out_i, np.int32), np.array(out_s, np.float64)


@pytest.mark.parametrize("seed", range(8))
def test_grouped_oracle_matches_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    S, T = int(rng.integers(9, 28)), int(rng.integers(3, 9))
    H, D = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    m = int(rng.integers(1, 4))
    g = int(rng.integers(1, 7))
    C = int(rng.integers(1, 6))
    topk = int(rng.integers(1, 6))
    off = int(rng.integers(0, 5))
    qb, w, kb = _case(rng, S, T, H, D)
    if seed % 2:   # gaussian-like values exercise the bfloat16 rounding of the mean
        qb = _bf16_bits(rng.standard_normal((S, H, D)).astype(np.float32))
        w = np.log1p(np.exp(rng.standard_normal((S, H)))).astype(np.float32)
    rows = np.arange(S, dtype=np.int64)
    got_i, got_s = oracle.grouped_rows(qb, w, kb, rows, m, topk, g, C, row_offset=off)
    want_i, want_s = _brute(qb, w, kb, rows, m, topk, g, C, row_offset=off)
    np.testing.assert_array_equal(got_i, want_i)
    np.testing.assert_allclose(got_s, want_s, rtol=1e-12, atol=0)


@pytest.mark.parametrize("g", [1, 4, 8, 16])
def test_grouped_equals_exact_when_candidates_cover_the_prefix(g):
    """C >= every visible count: each member scores all its visible keys,
    so the result is the exact oracle's, bit for bit."""
    rng = np.random.default_rng(g)
    S, T, H, D, m, topk = 200, 50, 8, 16, 4, 12
    qb, w, kb = _case(rng, S, T, H, D)
    rows = np.arange(S, dtype=np.int64)
    gi, gs = oracle.grouped_rows(qb, w, kb, rows, m, topk, g, T)
    ei, es = oracle.topk_rows(qb, w, kb, rows, m, topk)
    np.testing.assert_array_equal(gi, ei)
    np.testing.assert_array_equal(gs, es)


def test_groups_of_one_are_exact():
    """g = 1: the pooled query is the member's own (its bfloat16 mean of one
    value is itself), so the shared top-C (C >= k) holds its top-k."""
    rng = np.random.default_rng(5)
    S, T, H, D, m, topk = 300, 75, 4, 8, 4, 10
    qb = _bf16_bits(rng.standard_normal((S, H, D)).astype(np.float32))
    kb = _bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    w = np.abs(rng.standard_normal((S, H))).astype(np.float32)
    rows = np.arange(S, dtype=np.int64)
    gi, gs = oracle.grouped_rows(qb, w, kb, rows, m, topk, 1, topk)
    ei, es = oracle.topk_rows(qb, w, kb, rows, m, topk)
    np.testing.assert_array_equal(gi, ei)
    np.testing.assert_array_equal(gs, es)


def _recall(gi, ei):
    r = []
    for a, b in zip(gi, ei):
        sa, sb = set(a[a >= 0].tolist()), set(b[b >= 0].tolist())
        r.append(1.0 if not sb else len(sa & sb) / len(sb))
    return np.array(r)


def test_recall_monotone_in_candidates_and_outputs_valid():
    rng = np.random.default_rng(11)
    S, T, H, D, m, topk, g = 256, 64, 8, 16, 4, 8, 16
    qb = _bf16_bits(rng.standard_normal((S, H, D)).astype(np.float32))
    kb = _bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    w = np.log1p(np.exp(rng.standard_normal((S, H)))).astype(np.float32)
    rows = np.arange(S, dtype=np.int64)
    ei, _ = oracle.topk_rows(qb, w, kb, rows, m, topk)
    prev = None
    for C in (8, 12, 16, 24, 32, 64):
        gi, gs = oracle.grouped_rows(qb, w, kb, rows, m, topk, g, C)
        rec = _recall(gi, ei)
        if prev is not None:
            assert (rec >= prev - 1e-12).all()
        prev = rec
        # returned keys are visible, distinct, scored with the member's own score
        for r in rows:
            keys = gi[r][gi[r] >= 0]
            assert len(set(keys.tolist())) == len(keys)
            assert (keys < min(T, (r + 1) // m)).all()
            if len(keys):
                own = oracle.score_pairs(qb[r:r + 1], w[r:r + 1], kb,
                                         np.zeros(len(keys), np.int64), keys.astype(np.int64))
                np.testing.assert_array_equal(gs[r][:len(keys)], own)
                assert (np.diff(gs[r][:len(keys)]) <= 0).all()
    assert prev.min() == 1.0   # C = T: exact


@pytest.mark.parametrize("g,S", [(8, 64), (6, 40), (16, 37), (3, 10)])
def test_pooled_query_is_the_bf16_rounded_binary32_mean(g, S):
    """The pooling step against numpy float32 arithmetic in member order and
    torch's round-to-nearest-even cast to bfloat16, on every group, the
    short last one included."""
    rng = np.random.default_rng(g * 100 + S)
    H, D = 4, 32
    qb = _bf16_bits((rng.standard_normal((S, H, D)) * 3).astype(np.float32))
    w = np.abs(rng.standard_normal((S, H))).astype(np.float32)
    qv = _bf16_value(qb).astype(np.float32)
    for i0 in range(0, S, g):
        mem = range(i0, min(S, i0 + g))
        acc = np.zeros((H, D), np.float32)
        accw = np.zeros(H, np.float32)
        for u in mem:
            acc = (acc + qv[u]).astype(np.float32)
            accw = (accw + w[u]).astype(np.float32)
        want_q = _bf16_value(_bf16_bits(acc / np.float32(len(mem))))
        want_w = (accw / np.float32(len(mem))).astype(np.float64)
        for i in (i0, min(S, i0 + g) - 1):
            pq, pw = oracle.group_pool(qb, w, g, i)
            np.testing.assert_array_equal(pq, want_q)
            np.testing.assert_array_equal(pw, want_w)
