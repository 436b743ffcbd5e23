"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something fixed outside it: exact
rational brute force (a different selection algorithm: k rounds of argmax),
a hand-derived worked example, a library routine (numpy matmul + lexsort,
torch's bf16 / e4m3fn casts), closed forms and invariants of the
definition (StreamIndex: Memory-Bounded Compressed Sparse Attention via
Streaming Top-k, Abstract: lightning-indexer scores, the k best keys of each
query, and a chunk-by-chunk merge whose result equals the one-shot top-k).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def bf16_bits(values):
    """bf16 codes of values exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not representable in bf16"
    return (bits >> 16).astype(np.uint16)


def random_bf16_bits(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: still valid codes


def exact_bf16(bits):
    f = (np.asarray(bits, np.uint32) << 16).astype(np.uint32).view(np.float32)
    return np.vectorize(lambda x: Fraction(float(x)), otypes=[object])(f)


def exact_e4m3(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float32)
    return np.vectorize(lambda x: Fraction(float(x)), otypes=[object])(t.numpy())


def brute_force(qx, wx, kx, t, m, topk, qs=None, ks=None):
    """Exact rational scores and k rounds of argmax (first index wins ties)."""
    H, D = qx.shape
    T = kx.shape[0]
    n = min(T, max(0, (t + 1) // m))
    scores = []
    for s in range(n):
        tot = Fraction(0)
        for j in range(H):
            dot = sum((qx[j, x] * kx[s, x] for x in range(D)), Fraction(0))
            a = dot
            if qs is not None:
                a = Fraction(float(qs[j])) * Fraction(float(ks[s])) * dot
            if a > 0:
                tot += Fraction(float(wx[j])) * a
        scores.append(tot)
    chosen, left = [], list(range(n))
    for _ in range(min(topk, n)):
        best = left[0]
        for s in left[1:]:
            if scores[s] > scores[best]:
                best = s
        chosen.append(best)
        left.remove(best)
    idx = chosen + [-1] * (topk - len(chosen))
    sc = [scores[s] for s in chosen] + [None] * (topk - len(chosen))
    return idx, sc, scores


def run_oracle(q_bits, w, k_bits, t_rows, m, topk, dtype="bf16", **kw):
    return oracle.topk_rows(q_bits[t_rows], w[t_rows], k_bits, t_rows, m, topk, dtype=dtype, **kw)


# ---------------------------------------------------------------- decoding

def test_decode_bf16_all_codes(oracle_lib):
    codes = np.arange(1 << 16, dtype=np.uint32)
    ref = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_decode_e4m3fn_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3fn(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ---------------------------------------------------------------- worked example

def test_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    q = bf16_bits(np.array(g["q"], np.float32))
    k = bf16_bits(np.array(g["keys"], np.float32))
    w = np.array(g["w"], np.float32)
    t = np.arange(g["S"], dtype=np.int64)
    idx, sc = run_oracle(q, w, k, t, g["m"], g["k"])
    assert idx.tolist() == g["out_idx"]
    want = np.array([[-math.inf if v is None else v for v in row] for row in g["out_score"]])
    assert np.array_equal(sc, want)
    for tt in range(g["S"]):
        assert oracle.n_visible(tt, g["T"], g["m"]) == g["n_vis"][tt]
    rows = np.repeat(t, g["T"])
    keys = np.tile(np.arange(g["T"]), g["S"])
    allsc = oracle.score_pairs(q, w, k, rows, keys).reshape(g["S"], g["T"])
    assert np.array_equal(allsc, np.array(g["unmasked_scores"], np.float64))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("case", range(40))
def test_bruteforce_integer(oracle_lib, case):
    rng = np.random.default_rng(1000 + case)
    H = int(rng.choice([1, 2, 3, 4]))
    D = int(rng.integers(1, 9))
    m = int(rng.integers(1, 5))
    T = int(rng.integers(1, 17))
    S = int(rng.integers(1, m * T + 2 * m + 1))
    topk = int(rng.integers(1, T + 3))
    lo = -3 if case % 3 else -1  # small ranges -> many exact ties
    hi = 3 if case % 3 else 1
    qi = rng.integers(lo, hi + 1, (S, H, D)).astype(np.float32)
    ki = rng.integers(lo, hi + 1, (T, D)).astype(np.float32)
    w = rng.integers(0, 4, (S, H)).astype(np.float32)
    q_bits, k_bits = bf16_bits(qi), bf16_bits(ki)
    t = np.arange(S, dtype=np.int64)
    idx, sc = run_oracle(q_bits, w, k_bits, t, m, topk)
    for tt in range(S):
        bi, bs, _ = brute_force(qi[tt].astype(int).astype(object), w[tt], ki.astype(int).astype(object), tt, m, topk)
        assert idx[tt].tolist() == bi, (case, tt)
        for a, b in zip(sc[tt], bs):
            assert (a == -math.inf) if b is None else (a == float(b))


@pytest.mark.parametrize("case", range(12))
def test_bruteforce_random_bf16(oracle_lib, case):
    rng = np.random.default_rng(2000 + case)
    H, D = int(rng.integers(1, 5)), int(rng.integers(1, 7))
    m, T = int(rng.integers(1, 4)), int(rng.integers(2, 12))
    S = m * T + 1
    topk = int(rng.integers(1, T + 2))
    q_bits = random_bf16_bits(rng, (S, H, D))
    k_bits = random_bf16_bits(rng, (T, D))
    w = np.exp(rng.standard_normal((S, H))).astype(np.float32)
    t = np.arange(S, dtype=np.int64)
    idx, sc = run_oracle(q_bits, w, k_bits, t, m, topk)
    for tt in range(S):
        qx = exact_bf16(q_bits[tt])
        kx = exact_bf16(k_bits)
        bi, bs, allsc = brute_force(qx, w[tt], kx, tt, m, topk)
        vals = sorted(allsc, reverse=True)
        gaps = [abs(a - b) for a, b in zip(vals, vals[1:]) if a != 0 or b != 0]
        if gaps and min(gaps) < Fraction(1, 10 ** 9):
            continue  # a near tie double rounding could legally flip
        assert idx[tt].tolist() == bi
        for a, b in zip(sc[tt], bs):
            if b is None:
                assert a == -math.inf
            else:
                assert abs(a - float(b)) <= 1e-12 * max(1.0, abs(float(b)))


@pytest.mark.parametrize("case", range(10))
def test_bruteforce_fp8_scaled(oracle_lib, case):
    rng = np.random.default_rng(3000 + case)
    H, D = int(rng.integers(1, 4)), int(rng.integers(1, 6))
    m, T = int(rng.integers(1, 4)), int(rng.integers(2, 10))
    S = m * T + 2
    topk = int(rng.integers(1, T + 2))
    q_codes = rng.integers(0, 256, (S, H, D)).astype(np.uint8)
    k_codes = rng.integers(0, 256, (T, D)).astype(np.uint8)
    q_codes[(q_codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    k_codes[(k_codes & 0x7F) == 0x7F] = 0xB1
    qs = np.exp(rng.standard_normal((S, H))).astype(np.float32)
    ks = np.exp(rng.standard_normal(T)).astype(np.float32)
    w = rng.random((S, H)).astype(np.float32)
    t = np.arange(S, dtype=np.int64)
    idx, sc = oracle.topk_rows(q_codes, w, k_codes, t, m, topk, dtype="e4m3fn",
                               q_scale_rows=qs, k_scale=ks)
    kx = exact_e4m3(k_codes)
    for tt in range(S):
        bi, bs, allsc = brute_force(exact_e4m3(q_codes[tt]), w[tt], kx, tt, m, topk, qs=qs[tt], ks=ks)
        vals = sorted(allsc, reverse=True)
        gaps = [abs(a - b) for a, b in zip(vals, vals[1:]) if a != 0 or b != 0]
        if gaps and min(gaps) < Fraction(1, 10 ** 9):
            continue
        assert idx[tt].tolist() == bi
        for a, b in zip(sc[tt], bs):
            if b is None:
                assert a == -math.inf
            else:
                assert abs(a - float(b)) <= 1e-12 * max(1.0, abs(float(b)))


# ---------------------------------------------------------------- library special case

@pytest.mark.parametrize("m", [1, 2, 4])
def test_single_head_unit_weight_is_relu_dot_topk(oracle_lib, m):
    """H=1, w=1: the score is ReLU(q.k); compare with numpy float64 matmul
    and lexsort over the visible prefix."""
    rng = np.random.default_rng(7 + m)
    D, T, topk = 16, 40, 9
    S = m * T + 3
    q_bits = random_bf16_bits(rng, (S, 1, D))
    k_bits = random_bf16_bits(rng, (T, D))
    qf = (q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[:, 0, :]
    kf = (k_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = np.ones((S, 1), np.float32)
    t = np.arange(S, dtype=np.int64)
    idx, sc = run_oracle(q_bits, w, k_bits, t, m, topk)
    full = np.maximum(qf @ kf.T, 0.0)
    for tt in range(S):
        n = min(T, (tt + 1) // m)
        order = np.lexsort((np.arange(n), -full[tt, :n]))[:topk]
        want = list(order) + [-1] * (topk - len(order))
        assert idx[tt].tolist() == want
        np.testing.assert_allclose(sc[tt, :len(order)], full[tt, order], rtol=1e-12, atol=0)


# ---------------------------------------------------------------- invariants

def _case(seed, S=97, T=None, H=3, D=8, m=3, dist="gauss"):
    rng = np.random.default_rng(seed)
    T = T if T is not None else S // m
    if dist == "int":
        q_bits = bf16_bits(rng.integers(-2, 3, (S, H, D)).astype(np.float32))
        k_bits = bf16_bits(rng.integers(-2, 3, (T, D)).astype(np.float32))
        w = rng.integers(0, 3, (S, H)).astype(np.float32)
    else:
        q_bits = random_bf16_bits(rng, (S, H, D))
        k_bits = random_bf16_bits(rng, (T, D))
        w = np.exp(rng.standard_normal((S, H))).astype(np.float32)
    return q_bits, k_bits, w, np.arange(S, dtype=np.int64)


@pytest.mark.parametrize("dist", ["int", "gauss"])
def test_causality_and_padding(oracle_lib, dist):
    m, topk = 3, 7
    q, k, w, t = _case(11, m=m, dist=dist)
    T = k.shape[0]
    idx, sc = run_oracle(q, w, k, t, m, topk)
    # replacing every key a row cannot see leaves that row unchanged
    rng = np.random.default_rng(5)
    for tt in [0, 1, 2, 3, 10, 40, 96]:
        n = min(T, (tt + 1) // m)
        k2 = k.copy()
        k2[n:] = random_bf16_bits(rng, k2[n:].shape, scale=50.0)
        i2, s2 = run_oracle(q, w, k2, np.array([tt]), m, topk)
        assert np.array_equal(i2[0], idx[tt]) and np.array_equal(s2[0], sc[tt])
    for tt in range(len(t)):
        n = min(T, (tt + 1) // m)
        kept = min(topk, n)
        assert np.all(idx[tt, kept:] == -1) and np.all(sc[tt, kept:] == -np.inf)
        assert np.all((idx[tt, :kept] >= 0) & (idx[tt, :kept] < n))
        assert len(set(idx[tt, :kept].tolist())) == kept
        # sorted by (score desc, index asc)
        for a in range(kept - 1):
            assert sc[tt, a] > sc[tt, a + 1] or (sc[tt, a] == sc[tt, a + 1] and idx[tt, a] < idx[tt, a + 1])
        if kept == n:  # fewer visible keys than k: every visible key returned
            assert sorted(idx[tt, :kept].tolist()) == list(range(n))


@pytest.mark.parametrize("dist", ["int", "gauss"])
@pytest.mark.parametrize("chunk", [1, 3, 7, 16, 32])
def test_chunked_partition_merge_equals_full(oracle_lib, dist, chunk):
    m, topk = 3, 6
    q, k, w, t = _case(21, m=m, dist=dist)
    full = run_oracle(q, w, k, t, m, topk)
    part = run_oracle(q, w, k, t, m, topk, chunk=chunk)
    assert np.array_equal(full[0], part[0]) and np.array_equal(full[1], part[1])


def test_head_permutation_invariant(oracle_lib):
    q, k, w, t = _case(31, H=5)
    perm = np.array([3, 0, 4, 1, 2])
    a = run_oracle(q, w, k, t, 3, 5)
    b = run_oracle(q[:, perm], w[:, perm], k, t, 3, 5)
    assert np.array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)


def test_positive_weight_rescale_keeps_indices(oracle_lib):
    q, k, w, t = _case(41, dist="int")
    a = run_oracle(q, w, k, t, 3, 6)
    b = run_oracle(q, w * 4.0, k, t, 3, 6)  # exact power-of-two rescale
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(np.where(np.isfinite(a[1]), a[1] * 4.0, a[1]), b[1])


def test_negative_parts_clipped(oracle_lib):
    """Negating every key flips the sign of each head's dot product: with a
    single head, the keys that scored 0 now score |q.k| and vice versa."""
    q, k, w, t = _case(51, H=1, dist="int")
    kneg = bf16_bits(-((k.astype(np.uint32) << 16).view(np.float32)))
    T = k.shape[0]
    rows = np.repeat(t, T)
    keys = np.tile(np.arange(T), len(t))
    s_pos = oracle.score_pairs(q, w, k, rows, keys)
    s_neg = oracle.score_pairs(q, w, kneg, rows, keys)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[:, 0, :]
    kf = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dots = (qf @ kf.T).reshape(-1) * np.repeat(w[:, 0].astype(np.float64), T)
    assert np.array_equal(s_pos, np.maximum(dots, 0))
    assert np.array_equal(s_neg, np.maximum(-dots, 0))


def test_k_beyond_keys_and_empty_rows(oracle_lib):
    q, k, w, t = _case(61, S=20, T=5, m=2)
    idx, sc = run_oracle(q, w, k, t, 2, 9)
    assert np.all(idx[0] == -1)  # t=0 with m=2 sees nothing
    assert sorted(idx[19, :5].tolist()) == [0, 1, 2, 3, 4] and np.all(idx[19, 5:] == -1)


def test_materialized_tensor_closed_form():
    """Materialising every per-head score as fp32, [B,S,H_I,T] at S=65,536,
    H_I=64, m=4, takes 2**38 bytes = 256 GiB, the figure the abstract gives
    for it."""
    from csa_synth import WORKLOADS
    wl = WORKLOADS["s64k"]
    assert wl.B * wl.S * wl.H * wl.n_keys * 4 == 256 * 2 ** 30
