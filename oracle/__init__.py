"""Plain CPU oracle for the CSA lightning-indexer top-k step and the sparse
attention over the selected keys.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline may use this package; the product path never does.  It shares no
code with the HIP library.

The arithmetic lives in ``csa_oracle.c`` and ``csa_attn_oracle.c`` (plain C,
double precision); this module only builds them with gcc and marshals numpy
arrays through ctypes.

Definitions followed (StreamIndex: Memory-Bounded Compressed Sparse Attention
via Streaming Top-k, Abstract -- lightning indexer over compressed keys, top-k
per query): score(t, s) = sum_j w[t,j] * max(0, q[t,j,:] . k[s,:]) for the
visible keys s < min(T, floor((t+1)/m)); output the first min(k, n_vis) keys
by (score desc, index asc), padded with index -1 / score -inf.  Sparse
attention (same page and section: an attention kernel reads only the chosen
keys; no formula given): softmax(scale * q[t,h,:] . k[s,:]) over the valid
entries s of row t's index list, applied to v[s,:].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "csa_oracle.c"), os.path.join(_HERE, "csa_attn_oracle.c"),
         os.path.join(_HERE, "csa_group_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "libcsa_oracle.so")

DTYPE_CODES = {"bf16": 0, "e4m3fn": 1, "f32": 2}
_NP_STORAGE = {"bf16": np.uint16, "e4m3fn": np.uint8, "f32": np.float32}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libcsa_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
             "-o", tmp, *_SRCS, "-lpthread", "-lm"],
            check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.csa_oracle_rows.argtypes = [p, i32, p, p, p, i32, p, p, i64, i64, i32,
                                    i32, i32, i32, i64, i32, p, p]
    lib.csa_oracle_rows.restype = i32
    lib.csa_oracle_score_pairs.argtypes = [p, i32, p, p, p, i32, p, i64, i32,
                                           i32, p, p, i64, p]
    lib.csa_oracle_score_pairs.restype = i32
    lib.csa_oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.csa_oracle_decode_bf16.restype = ctypes.c_double
    lib.csa_oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.csa_oracle_decode_e4m3fn.restype = ctypes.c_double
    lib.csa_oracle_n_visible.argtypes = [i64, i64, i32]
    lib.csa_oracle_n_visible.restype = i64
    lib.csa_oracle_sparse_attention.argtypes = [p, p, p, p, i64, i64, i32, i32, i32,
                                                ctypes.c_double, i32, p, p, p]
    lib.csa_oracle_sparse_attention.restype = i32
    lib.csa_oracle_grouped.argtypes = [p, p, p, i64, i64, i32, i32, i32, i32, i32, i32, i64, p,
                                       i64, i32, p, p]
    lib.csa_oracle_grouped.restype = i32
    lib.csa_oracle_group_pool.argtypes = [p, p, i64, i32, i32, i32, i64, p, p]
    lib.csa_oracle_group_pool.restype = i64
    _lib = lib
    return lib


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _opt(a):
    if a is None:
        return None, None
    return _arr(a, np.float32)


def decode_bf16(bits: int) -> float:
    return _load().csa_oracle_decode_bf16(int(bits))


def decode_e4m3fn(bits: int) -> float:
    return _load().csa_oracle_decode_e4m3fn(int(bits))


def n_visible(t: int, T: int, m: int) -> int:
    return int(_load().csa_oracle_n_visible(int(t), int(T), int(m)))


def topk_rows(q_rows, w_rows, k_keys, t_rows, m, topk, *, dtype="bf16",
              q_scale_rows=None, k_scale=None, chunk=0, nthreads=None):
    """Top-k for the query positions ``t_rows``.

    q_rows: [n, H, D] storage of the requested rows (uint16 bf16 bits, uint8
    e4m3fn bits or float32, per ``dtype``); w_rows: [n, H] float32;
    k_keys: [T, D] same storage as q; q_scale_rows: [n, H] / k_scale: [T]
    float32 per-row scales (fp8) or None.  Returns (idx int32 [n, k],
    score float64 [n, k]).
    """
    lib = _load()
    store = _NP_STORAGE[dtype]
    q_rows, qp = _arr(q_rows, store)
    k_keys, kp = _arr(k_keys, store)
    w_rows, wp = _arr(w_rows, np.float32)
    t_rows, tp = _arr(t_rows, np.int64)
    qs, qsp = _opt(q_scale_rows)
    ks, ksp = _opt(k_scale)
    n, H, D = q_rows.shape
    T = k_keys.shape[0]
    assert k_keys.shape[1] == D and w_rows.shape == (n, H) and t_rows.shape == (n,)
    out_idx = np.empty((n, topk), np.int32)
    out_score = np.empty((n, topk), np.float64)
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = lib.csa_oracle_rows(qp, DTYPE_CODES[dtype], qsp, wp, kp, DTYPE_CODES[dtype],
                             ksp, tp, n, T, H, D, int(m), int(topk), int(chunk),
                             int(nthreads), out_idx.ctypes.data_as(ctypes.c_void_p),
                             out_score.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise RuntimeError("csa_oracle_rows failed")
    return out_idx, out_score


def grouped_rows(q_entry, w_entry, k_keys, rows, m, topk, group, candidates, *, row_offset=0,
                 nthreads=None):
    """The grouped (approximate) top-k of rows ``rows`` of one batch entry
    (csa_group_oracle.c): q_entry [S, H, D] bf16 bits (uint16) and w_entry
    [S, H] float32 for every row of the entry, k_keys [T, D] bf16 bits.
    Returns (idx int32 [n, k], score float64 [n, k])."""
    lib = _load()
    q_entry, qp = _arr(q_entry, np.uint16)
    w_entry, wp = _arr(w_entry, np.float32)
    k_keys, kp = _arr(k_keys, np.uint16)
    rows, rp = _arr(rows, np.int64)
    S, H, D = q_entry.shape
    T = k_keys.shape[0]
    n = rows.shape[0]
    out_idx = np.empty((n, topk), np.int32)
    out_score = np.empty((n, topk), np.float64)
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = lib.csa_oracle_grouped(qp, wp, kp, S, T, H, D, int(m), int(topk), int(group),
                                int(candidates), int(row_offset), rp, n, int(nthreads),
                                out_idx.ctypes.data_as(ctypes.c_void_p),
                                out_score.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise RuntimeError("csa_oracle_grouped failed")
    return out_idx, out_score


def group_pool(q_entry, w_entry, group, row):
    """The pooled query of the group holding ``row`` (csa_group_oracle.c):
    (pq float64 [H, D] bfloat16 values, pw float64 [H])."""
    lib = _load()
    q_entry, qp = _arr(q_entry, np.uint16)
    w_entry, wp = _arr(w_entry, np.float32)
    S, H, D = q_entry.shape
    pq = np.empty((H, D), np.float64)
    pw = np.empty(H, np.float64)
    lib.csa_oracle_group_pool(qp, wp, S, H, D, int(group), int(row),
                              pq.ctypes.data_as(ctypes.c_void_p), pw.ctypes.data_as(ctypes.c_void_p))
    return pq, pw


def score_pairs(q_rows, w_rows, k_keys, row, key, *, dtype="bf16",
                q_scale_rows=None, k_scale=None):
    """Scores (float64) of (row, key) pairs, visibility ignored."""
    lib = _load()
    store = _NP_STORAGE[dtype]
    q_rows, qp = _arr(q_rows, store)
    k_keys, kp = _arr(k_keys, store)
    w_rows, wp = _arr(w_rows, np.float32)
    qs, qsp = _opt(q_scale_rows)
    ks, ksp = _opt(k_scale)
    row, rp = _arr(row, np.int64)
    key, kyp = _arr(key, np.int64)
    n, H, D = q_rows.shape
    T = k_keys.shape[0]
    out = np.empty(row.shape[0], np.float64)
    rc = lib.csa_oracle_score_pairs(qp, DTYPE_CODES[dtype], qsp, wp, kp,
                                    DTYPE_CODES[dtype], ksp, T, H, D, rp, kyp,
                                    row.shape[0], out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise RuntimeError("csa_oracle_score_pairs failed")
    return out


def sparse_attention(q_rows, k_keys, v_keys, idx_rows, scale, *, nthreads=None,
                     with_bound=True):
    """Softmax attention of each query row over its selected compressed keys.

    q_rows: [n, H, D] bf16 bits (uint16) of the requested rows; k_keys,
    v_keys: [T, D] bf16 bits; idx_rows: [n, L] int32 index lists, entries
    outside [0, T) are padding.  Returns (o float64 [n, H, D], lse float64
    [n, H], a float64 [n, H, D] or None), where a is the softmax-weighted
    magnitude sum_e p_e |v_e| that bounds rounding in the weights.
    """
    lib = _load()
    q_rows, qp = _arr(q_rows, np.uint16)
    k_keys, kp = _arr(k_keys, np.uint16)
    v_keys, vp = _arr(v_keys, np.uint16)
    idx_rows, ip = _arr(idx_rows, np.int32)
    n, H, D = q_rows.shape
    T = k_keys.shape[0]
    assert v_keys.shape == (T, D) and k_keys.shape[1] == D and idx_rows.shape[0] == n
    L = idx_rows.shape[1]
    o = np.empty((n, H, D), np.float64)
    lse = np.empty((n, H), np.float64)
    a = np.empty((n, H, D), np.float64) if with_bound else None
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = lib.csa_oracle_sparse_attention(
        qp, kp, vp, ip, n, T, H, D, L, float(scale), int(nthreads),
        o.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p),
        a.ctypes.data_as(ctypes.c_void_p) if a is not None else None)
    if rc != 0:
        raise RuntimeError("csa_oracle_sparse_attention failed")
    return o, lse, a
