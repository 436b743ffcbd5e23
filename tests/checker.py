"""Comparison of GPU top-k rows against the CPU oracle (test infrastructure).

Acceptance, per the indexer's definition (StreamIndex: Memory-Bounded
Compressed Sparse Attention via Streaming Top-k, Abstract: the k best keys
of each query, measured by how much of the exact top-k set is recovered):

* exact inputs (integer-valued, every fp32 partial sum exact): indices and
  scores identical to the oracle, element by element;
* floating-point inputs: the same number of kept keys and identical padding;
  every key in the symmetric difference of the two top-k sets scores, by the
  oracle's fp64 definition, within ``rtol`` (1e-3) of the oracle's k-th
  score (recall 1.0 up to such near-ties); each returned score is within
  ``rtol`` of that key's fp64 score; the GPU row is ordered by its own scores
  (descending, ties by ascending index); returned keys are visible and
  distinct.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from csa_synth import storage_numpy


class OracleView:
    """Host copies of the inputs of one batch entry, for the oracle."""

    def __init__(self, inp, wl, b=0):
        self.wl = wl
        self.dtype = wl.dtype
        self.q = inp["q"][b]
        self.w = inp["w"][b]
        self.k = storage_numpy(inp["k"][b])
        self.qs = inp.get("q_scale")
        self.ks = inp.get("k_scale")
        self.qs = self.qs[b] if self.qs is not None else None
        self.ks = self.ks[b].cpu().numpy() if self.ks is not None else None

    def rows(self, rows):
        rt = torch.as_tensor(np.asarray(rows), device=self.q.device)
        q = storage_numpy(self.q.index_select(0, rt))
        w = self.w.index_select(0, rt).cpu().numpy()
        qs = self.qs.index_select(0, rt).cpu().numpy() if self.qs is not None else None
        return q, w, qs

    def topk(self, rows, t_rows, k, m, chunk=0):
        q, w, qs = self.rows(rows)
        return oracle.topk_rows(q, w, self.k, t_rows, m, k, dtype=self.dtype,
                                q_scale_rows=qs, k_scale=self.ks, chunk=chunk)

    def score(self, rows, row_of_pair, key_of_pair):
        q, w, qs = self.rows(rows)
        return oracle.score_pairs(q, w, self.k, row_of_pair, key_of_pair, dtype=self.dtype,
                                  q_scale_rows=qs, k_scale=self.ks)


def compare_exact(g_idx, g_score, o_idx, o_score, t_rows=None):
    g_idx = np.asarray(g_idx)
    g_score = np.asarray(g_score, dtype=np.float64)
    bad = np.nonzero(np.any(g_idx != o_idx, axis=1) | np.any(g_score != o_score, axis=1))[0]
    if bad.size:
        r = bad[0]
        where = f"t={t_rows[r]}" if t_rows is not None else f"row {r}"
        j = int(np.nonzero((g_idx[r] != o_idx[r]) | (g_score[r] != o_score[r]))[0][0])
        raise AssertionError(
            f"{bad.size} rows differ; first at {where}, slot {j}: gpu ({g_idx[r, j]}, "
            f"{g_score[r, j]}) vs oracle ({o_idx[r, j]}, {o_score[r, j]})")


def compare_tolerant(g_idx, g_score, o_idx, o_score, score_fn, t_rows, T, m, rtol=1e-3):
    """score_fn(row_of_pair, key_of_pair) -> fp64 oracle scores of pairs."""
    g_idx = np.asarray(g_idx)
    g_score = np.asarray(g_score, dtype=np.float64)
    nrows, k = o_idx.shape
    pair_r, pair_k = [], []
    for r in range(nrows):
        n_vis = min(T, (int(t_rows[r]) + 1) // m)
        kept = int(np.sum(o_idx[r] >= 0))
        assert kept == min(k, n_vis), (t_rows[r], kept, n_vis)
        gk = g_idx[r, :kept]
        assert np.all(g_idx[r, kept:] == -1), f"t={t_rows[r]}: padding indices"
        assert np.all(np.isneginf(g_score[r, kept:])), f"t={t_rows[r]}: padding scores"
        assert np.all((gk >= 0) & (gk < n_vis)), f"t={t_rows[r]}: invisible key returned"
        assert np.unique(gk).size == kept, f"t={t_rows[r]}: duplicate keys"
        gs = g_score[r, :kept]
        order_ok = (gs[:-1] > gs[1:]) | ((gs[:-1] == gs[1:]) & (gk[:-1] < gk[1:]))
        assert np.all(order_ok), f"t={t_rows[r]}: row not sorted by (score desc, index asc)"
        pair_r.append(np.full(kept, r))
        pair_k.append(gk)
    if not pair_r:
        return {"max_rel_err": 0.0, "swaps": 0, "recall": 1.0, "recall_min": 1.0}
    pr = np.concatenate(pair_r)
    pk = np.concatenate(pair_k)
    s_true = score_fn(pr, pk)
    swaps = 0
    max_rel = 0.0
    off = 0
    hits = total = 0          # set overlap |G & O| over min(k, n_vis), pooled
    recall_min = 1.0
    for r in range(nrows):
        kept = int(np.sum(o_idx[r] >= 0))
        if kept == 0:
            continue
        s_k = o_score[r, kept - 1]
        st = s_true[off:off + kept]
        gs = g_score[r, :kept]
        scale = np.maximum(np.abs(st), abs(s_k))
        err = np.abs(gs - st)
        ok = err <= rtol * scale
        assert np.all(ok), (f"t={t_rows[r]}: returned score off by "
                            f"{float(np.max(err / np.where(scale > 0, scale, 1)))} relative")
        if np.any(scale > 0):
            max_rel = max(max_rel, float(np.max(err[scale > 0] / scale[scale > 0])))
        gset = set(g_idx[r, :kept].tolist())
        oset = set(o_idx[r, :kept].tolist())
        common = len(gset & oset)
        hits += common
        total += kept
        recall_min = min(recall_min, common / kept)
        diff = gset ^ oset
        if diff:
            swaps += len(diff) // 2
            keys = np.array(sorted(diff), dtype=np.int64)
            sd = score_fn(np.full(keys.size, r), keys)
            if s_k == 0:
                assert np.all(sd == 0), f"t={t_rows[r]}: swapped keys with nonzero score"
            else:
                rel = np.abs(sd - s_k) / abs(s_k)
                assert np.all(rel <= rtol), (f"t={t_rows[r]}: swapped key {keys[np.argmax(rel)]} "
                                             f"is {float(rel.max())} from the k-th score")
        off += kept
    return {"max_rel_err": max_rel, "swaps": swaps,
            "recall": hits / total if total else 1.0, "recall_min": recall_min}


# ------------------------------------------------------------ sparse attention

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_reference(inp, b, rows, scale):
    """Oracle outputs for rows `rows` of batch entry b of an attention input
    dict (q, k, v, idx on any device), plus the bound on the score error.

    Score error: each q.k is an fp32 sum of D exact bf16 products, whatever
    the summation order within D*2^-24 * sum_x |q_x k_x|, which is at most
    D*2^-24 * |q| |k| (Cauchy-Schwarz); dz is that times |scale|, maximised
    over the row's valid entries.
    """
    q = storage_numpy(inp["q"][b, torch.as_tensor(rows, device=inp["q"].device)])
    k = storage_numpy(inp["k"][b])
    v = storage_numpy(inp["v"][b])
    idx = inp["idx"][b, torch.as_tensor(rows, device=inp["idx"].device)].cpu().numpy()
    o, lse, a = oracle.sparse_attention(q, k, v, idx, scale)
    T, D = k.shape
    qn = np.linalg.norm(bf16_to_f64(q), axis=-1)                       # [n, H]
    kn = np.linalg.norm(bf16_to_f64(k), axis=-1) if T > 0 else np.zeros(0)
    valid = (idx >= 0) & (idx < T)
    kmax = np.array([kn[r[v_]].max() if v_.any() else 0.0 for r, v_ in zip(idx, valid)])
    dz = abs(scale) * D * 2.0 ** -24 * qn * kmax[:, None]              # [n, H]
    return o, lse, a, dz


def compare_attention(g_out, g_lse, o, lse, a, dz):
    """GPU rows (bf16 out [n,H,D] as uint16 bits, fp32 lse [n,H]) against
    the oracle.  Bound per element, from the kernel's arithmetic:
      * weights rounded to bf16 for the value sum: <= 2^-9 * a, with
        a = sum_e p_e |v_e| (the normaliser uses unrounded weights);
      * score error dz moves o by at most 2 * dz * a (d o / d z_e =
        p_e (v_e - o));
      * fp32 accumulation and the final bf16 rounding: <= 2^-9 * |o| plus
        terms far below the first;
    so |out - o| <= 2^-8 * (a + |o|) + 2 * dz * a (a factor 2 of margin on
    the rounding terms).  lse: |lse' - lse| <= dz + 2^-20 * (1 + |lse|).
    Rows without valid entries must be exactly 0 with lse = -inf.
    """
    out = bf16_to_f64(g_out)
    empty = np.isneginf(lse)
    assert np.array_equal(np.isneginf(g_lse), empty), "empty rows differ"
    assert np.all(out[empty] == 0), "empty rows must be zero"
    tol = 2.0 ** -8 * (a + np.abs(o)) + 2 * dz[..., None] * a
    err = np.abs(out - o)
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} elements out of bound; worst excess "
                           f"{(err - tol).max():.3e} at {np.unravel_index((err - tol).argmax(), err.shape)}")
    fin = ~empty
    ltol = dz[fin] + 2.0 ** -20 * (1 + np.abs(lse[fin]))
    lerr = np.abs(g_lse[fin].astype(np.float64) - lse[fin])
    assert np.all(lerr <= ltol), f"lse off by {lerr.max():.3e}"
    rel = err[fin] / np.maximum(a[fin], 1e-30)
    return {"max_err_over_a": float(rel.max()) if rel.size else 0.0,
            "max_lse_err": float(lerr.max()) if lerr.size else 0.0}
