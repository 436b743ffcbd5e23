"""Pins for the sparse-attention oracle, independent of the oracle's code.

The oracle computes softmax attention of each query head over the keys its
index list selects (StreamIndex: Memory-Bounded Compressed Sparse Attention
via Streaming Top-k, Abstract: the attention after the indexer reads only
the chosen keys).  Each test checks it against something fixed outside it:
a hand-derived example, torch's float64 scaled_dot_product_attention and
logsumexp (library routines) on lists that hold every visible key, closed
forms (one entry, equal scores, no entry) and invariances of the definition
(order of the list, padding, head permutation, linearity in v).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(values):
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not representable in bf16"
    return (bits >> 16).astype(np.uint16)


def random_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def as_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _val(x):
    if isinstance(x, (int, float)):
        return float(x)
    table = {"ln7": math.log(7), "ln3": math.log(3), "ln2": math.log(2), "0": 0.0,
             "-inf": -math.inf}
    if x in table:
        return table[x]
    num, den = x.split("/")
    return int(num) / int(den)


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_example.json")))
    q = bf16_bits(g["q"])
    k = bf16_bits(g["keys"])
    v = bf16_bits(g["values"])
    idx = np.array(g["idx"], np.int32)
    o, lse, a = oracle.sparse_attention(q, k, v, idx, math.log(2))
    want_o = np.array([[[_val(x) for x in hv] for hv in row] for row in g["o"]])
    want_lse = np.array([[_val(x) for x in row] for row in g["lse"]])
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(want_lse))
    fin = np.isfinite(want_lse)
    np.testing.assert_allclose(lse[fin], want_lse[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a, np.abs(want_o), atol=1e-12)  # v >= 0 here


@pytest.mark.parametrize("T,H,D,m,seed", [(40, 3, 16, 2, 0), (100, 8, 64, 4, 1), (9, 1, 8, 1, 2)])
def test_matches_torch_sdpa_on_full_lists(T, H, D, m, seed):
    """Lists holding every causally visible key (shuffled, padded with -1 and
    an out-of-range index) reduce the method to masked dense attention."""
    rng = np.random.default_rng(seed)
    S = m * T
    q = random_bf16(rng, (S, H, D))
    k = random_bf16(rng, (T, D))
    v = random_bf16(rng, (T, D))
    L = T + 5
    idx = np.full((S, L), -1, np.int32)
    for t in range(S):
        n = min(T, (t + 1) // m)
        slots = rng.permutation(L)[:n + 1]
        idx[t, slots[:n]] = rng.permutation(n)
        idx[t, slots[n]] = T + 3 if n < L else -1  # beyond the keys: padding
    scale = 1.0 / math.sqrt(D) * 1.3
    o, lse, a = oracle.sparse_attention(q, k, v, idx, scale)

    qt = torch.from_numpy(as_f64(q)).permute(1, 0, 2)          # [H, S, D]
    kt = torch.from_numpy(as_f64(k))[None].expand(H, T, D)
    vt = torch.from_numpy(as_f64(v))[None].expand(H, T, D)
    t_pos = torch.arange(S)[:, None]
    s_pos = torch.arange(T)[None, :]
    mask = (s_pos + 1) * m - 1 <= t_pos                         # [S, T]
    has = mask.any(dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt[:, has], kt, vt, attn_mask=mask[has], scale=scale)
    z = torch.einsum("hsd,htd->hst", qt, kt) * scale
    ref_lse = torch.logsumexp(z.masked_fill(~mask, -math.inf), dim=-1)  # [H, S]
    got = torch.from_numpy(o).permute(1, 0, 2)
    torch.testing.assert_close(got[:, has], ref, rtol=1e-10, atol=1e-12)
    assert torch.all(got[:, ~has] == 0)
    torch.testing.assert_close(torch.from_numpy(lse).T[:, has], ref_lse[:, has],
                               rtol=1e-12, atol=1e-12)
    assert np.all(np.isneginf(lse[~has.numpy()]))
    assert np.all(a >= np.abs(o) - 1e-12)


def test_single_entry_is_that_value():
    rng = np.random.default_rng(5)
    T, H, D = 30, 4, 32
    q = random_bf16(rng, (T, H, D))
    k = random_bf16(rng, (T, D))
    v = random_bf16(rng, (T, D))
    idx = np.full((T, 6), -1, np.int32)
    keys = rng.integers(0, T, size=T)
    idx[np.arange(T), rng.integers(0, 6, size=T)] = keys
    o, lse, _ = oracle.sparse_attention(q, k, v, idx, 0.7)
    vd, kd, qd = as_f64(v), as_f64(k), as_f64(q)
    for t in range(T):
        np.testing.assert_array_equal(o[t], np.broadcast_to(vd[keys[t]], (H, D)))
        np.testing.assert_allclose(lse[t], 0.7 * qd[t] @ kd[keys[t]], rtol=1e-13)


def test_equal_scores_average_the_values():
    """scale = 0 makes every weight equal: o is the mean of the selected
    values and lse = log(number of valid entries)."""
    rng = np.random.default_rng(6)
    T, H, D, L = 50, 2, 16, 12
    q = random_bf16(rng, (7, H, D))
    k = random_bf16(rng, (T, D))
    v = random_bf16(rng, (T, D))
    idx = np.stack([rng.choice(np.r_[np.arange(T), [-1] * 5], size=L, replace=False)
                    for _ in range(7)]).astype(np.int32)
    o, lse, _ = oracle.sparse_attention(q, k, v, idx, 0.0)
    vd = as_f64(v)
    for r in range(7):
        sel = idx[r][idx[r] >= 0]
        np.testing.assert_allclose(o[r], np.broadcast_to(vd[sel].mean(0), (H, D)), atol=1e-14)
        np.testing.assert_allclose(lse[r], math.log(len(sel)), atol=1e-14)


def test_empty_lists_and_no_keys():
    rng = np.random.default_rng(7)
    q = random_bf16(rng, (3, 2, 8))
    k = random_bf16(rng, (4, 8))
    v = random_bf16(rng, (4, 8))
    idx = np.array([[-1, -1], [4, 9], [-5, -1]], np.int32)
    o, lse, a = oracle.sparse_attention(q, k, v, idx, 1.0)
    assert np.all(o == 0) and np.all(a == 0) and np.all(np.isneginf(lse))
    o, lse, _ = oracle.sparse_attention(q, np.zeros((0, 8), np.uint16),
                                        np.zeros((0, 8), np.uint16), idx, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse, _ = oracle.sparse_attention(q, k, v, np.zeros((3, 0), np.int32), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_invariances():
    """Reordering the list and moving the padding change nothing; permuting
    the heads of q permutes the output heads; o is linear in v."""
    rng = np.random.default_rng(8)
    n, T, H, D, L = 9, 64, 6, 32, 20
    q = random_bf16(rng, (n, H, D))
    k = random_bf16(rng, (T, D))
    v = random_bf16(rng, (T, D))
    idx = np.stack([np.r_[rng.choice(T, size=L - 4, replace=False), [-1] * 4]
                    for _ in range(n)]).astype(np.int32)
    o, lse, _ = oracle.sparse_attention(q, k, v, idx, 0.2)

    shuffled = np.stack([rng.permutation(r) for r in idx]).astype(np.int32)
    o2, lse2, _ = oracle.sparse_attention(q, k, v, shuffled, 0.2)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)

    perm = rng.permutation(H)
    o3, lse3, _ = oracle.sparse_attention(q[:, perm], k, v, idx, 0.2)
    np.testing.assert_array_equal(o3, o[:, perm])
    np.testing.assert_array_equal(lse3, lse[:, perm])

    v2 = ((v.astype(np.uint32) + (1 << 7)) & 0xFFFF).astype(np.uint16)  # exponent + 1: 2 * v
    finite = np.abs(as_f64(v)) < 1e30
    assert np.all(finite)
    np.testing.assert_array_equal(as_f64(v2)[as_f64(v) != 0], 2 * as_f64(v)[as_f64(v) != 0])
    v2[as_f64(v) == 0] = v[as_f64(v) == 0]
    o4, _, _ = oracle.sparse_attention(q, k, v2, idx, 0.2)
    np.testing.assert_allclose(o4, 2 * o, rtol=1e-12, atol=1e-13)
