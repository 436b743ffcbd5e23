"""Seeded synthetic inputs for the CSA lightning-indexer step and for the
sparse attention over the selected keys.

This module only draws random numbers and lays them out; it holds none of
the indexer's or the attention's arithmetic (no scoring, no selection, no
softmax).  Both the HIP path and
the CPU oracle consume the tensors it produces, bit for bit.

The workloads are V4-shaped indexer inputs (StreamIndex: Memory-Bounded
Compressed Sparse Attention via Streaming Top-k, Abstract: synthetic inputs;
the indexer has H_I = 64 heads and the keys are compressed by m = 4).
The distributions below are the ones the benchmark configurations name:

* ``int``   : q and k integers uniform in [-3, 3], w integers uniform in
              [0, 3].  Every fp32 partial sum is an integer below 2**24, so
              results are exact.
* ``gauss`` : q ~ N(0, 1); k = (0.5 * (Z @ V) / sqrt(8) + E) / sqrt(D) with
              Z [T, 8], V [8, D], E [T, D] ~ N(0, 1) (a shared rank-8
              component plus noise); w = softplus(N(0, 1)).
* ``gauss`` with ``q_rho`` > 0 (a sensitivity input for the grouped
              indexer, not a benchmark configuration): q[t] =
              sqrt(rho) * U[t // q_seg] + sqrt(1 - rho) * N(0, 1), with one
              N(0, 1) row U per segment of q_seg consecutive positions, so
              positions of one segment are correlated with coefficient rho
              (every entry still N(0, 1)); k and w as ``gauss``.

q and k are stored as bf16, or as OCP e4m3fn with one positive fp32 scale
per row (per (t, head) row of q, per key of k): scale = amax / 448, values
divided by the scale, clamped to +-448 and rounded to nearest even by the
cast.  Integer inputs are stored in fp8 with scale 1.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

FP8_MAX = 448.0
_ROW_CHUNK = 8192  # rows drawn per generator call (fixed: keeps streams stable)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    m: int
    H: int
    D: int
    k: int
    dist: str = "gauss"     # "int" | "gauss"
    dtype: str = "bf16"     # "bf16" | "e4m3fn"
    T: int = -1             # -1: S // m
    row_offset: int = 0     # absolute position of q row 0
    q_rho: float = 0.0      # gauss: correlation of q rows within a segment
    q_seg: int = 64         # positions per segment (q_rho > 0)

    @property
    def n_keys(self) -> int:
        return self.T if self.T >= 0 else self.S // self.m

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny-int": Workload("tiny-int", B=1, S=1024, m=4, H=4, D=32, k=64, dist="int"),
    "s16k": Workload("s16k", B=1, S=16384, m=4, H=64, D=128, k=512),
    "s64k": Workload("s64k", B=1, S=65536, m=4, H=64, D=128, k=2048),
    "s256k": Workload("s256k", B=1, S=262144, m=4, H=64, D=128, k=2048),
    "s256k-int": Workload("s256k-int", B=1, S=262144, m=4, H=64, D=128, k=2048, dist="int"),
    "s1m-fp8": Workload("s1m-fp8", B=1, S=1048576, m=4, H=64, D=128, k=2048, dtype="e4m3fn"),
    "s1m-fp8-int": Workload("s1m-fp8-int", B=1, S=1048576, m=4, H=64, D=128, k=2048,
                            dist="int", dtype="e4m3fn"),
    # short query blocks at the end of a long context (a decode step, or the
    # last rows of a chunked prefill): 64 positions after 262,080 others, and
    # 32 sequences with 4 new positions each after 65,532
    "dec64": Workload("dec64", B=1, S=64, m=4, H=64, D=128, k=2048, T=65536,
                      row_offset=4 * 65536 - 64),
    "dec64-int": Workload("dec64-int", B=1, S=64, m=4, H=64, D=128, k=2048, T=65536,
                          row_offset=4 * 65536 - 64, dist="int"),
    "dec32x4": Workload("dec32x4", B=32, S=4, m=4, H=64, D=128, k=2048, T=16384,
                        row_offset=4 * 16384 - 4),
}

# chunk sizes (compressed keys) and top-k values swept on the S = 65,536
# workload, five points around its defaults (chunk 8192, k 2048)
CHUNK_SWEEP = (1024, 2048, 4096, 8192, 16384)
TOPK_SWEEP = (256, 512, 1024, 2048, 4096)
# keys staged per LDS tile, and keys per key range (the partition of the T
# keys whose exact top-k lists are merged), on the same workload
KEY_TILE_SWEEP = (32, 64, 128, 192, 256)
RANGE_SWEEP = (1024, 2048, 4096, 8192, 16384)


def _generator(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + stream)
    return g


def _draw(shape, kind, gen, device):
    if kind == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if kind == "int3":
        return torch.randint(-3, 4, shape, generator=gen, device=device).to(torch.float32)
    if kind == "int0_3":
        return torch.randint(0, 4, shape, generator=gen, device=device).to(torch.float32)
    raise ValueError(kind)


def _rows(nrows, row_shape, kind, gen, device, sink):
    """Draw nrows rows in fixed-size pieces; sink(r0, r1, fp32 piece)."""
    for r0 in range(0, nrows, _ROW_CHUNK):
        r1 = min(nrows, r0 + _ROW_CHUNK)
        sink(r0, r1, _draw((r1 - r0,) + tuple(row_shape), kind, gen, device))


def _fp8_rows(x):
    """Per-row (last axis) scale and e4m3fn codes of an fp32 tensor."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale.to(torch.float32)


def make_inputs(wl: Workload, seed: int = 0, device="cpu"):
    """Tensors q [B,S,H,D], w [B,S,H] fp32, k [B,T,D] (+ q_scale [B,S,H],
    k_scale [B,T] for fp8) on ``device``.  Deterministic per (wl, seed,
    device type)."""
    B, S, H, D, T = wl.B, wl.S, wl.H, wl.D, wl.n_keys
    fp8 = wl.dtype == "e4m3fn"
    store = torch.float8_e4m3fn if fp8 else torch.bfloat16
    q = torch.empty((B, S, H, D), dtype=store, device=device)
    w = torch.empty((B, S, H), dtype=torch.float32, device=device)
    k = torch.empty((B, T, D), dtype=store, device=device)
    q_scale = torch.empty((B, S, H), dtype=torch.float32, device=device) if fp8 else None
    k_scale = torch.empty((B, T), dtype=torch.float32, device=device) if fp8 else None
    integer = wl.dist == "int"

    for b in range(B):
        gq = _generator(device, seed, 10 * b + 1)
        gw = _generator(device, seed, 10 * b + 2)
        gk = _generator(device, seed, 10 * b + 3)

        useg = None
        if wl.q_rho > 0 and not integer:
            useg = _draw(((S + wl.q_seg - 1) // wl.q_seg, H, D), "normal",
                         _generator(device, seed, 10 * b + 4), device)

        def put_q(r0, r1, x, b=b, useg=useg):
            if useg is not None:
                seg = torch.arange(r0, r1, device=x.device) // wl.q_seg
                x = (float(np.sqrt(1.0 - wl.q_rho)) * x +
                     float(np.sqrt(wl.q_rho)) * useg.index_select(0, seg))
            if fp8 and not integer:
                codes, sc = _fp8_rows(x)
                q[b, r0:r1] = codes
                q_scale[b, r0:r1] = sc
            else:
                q[b, r0:r1] = x.to(store)
                if fp8:
                    q_scale[b, r0:r1] = 1.0

        _rows(S, (H, D), "int3" if integer else "normal", gq, device, put_q)

        def put_w(r0, r1, x, b=b):
            w[b, r0:r1] = x if integer else torch.nn.functional.softplus(x)

        _rows(S, (H,), "int0_3" if integer else "normal", gw, device, put_w)

        if integer:
            kf = _draw((T, D), "int3", gk, device)
        else:
            z = _draw((T, 8), "normal", gk, device)
            v = _draw((8, D), "normal", gk, device)
            e = _draw((T, D), "normal", gk, device)
            kf = (0.5 * (z @ v) / np.sqrt(8.0) + e) / np.sqrt(float(D))
        if fp8 and not integer:
            codes, sc = _fp8_rows(kf)
            k[b] = codes
            k_scale[b] = sc
        else:
            k[b] = kf.to(store)
            if fp8:
                k_scale[b] = 1.0
    out = {"q": q, "w": w, "k": k}
    if fp8:
        out["q_scale"] = q_scale
        out["k_scale"] = k_scale
    return out


def sample_rows(S: int, m: int, topk: int, n: int = 256, seed: int = 0, chunk: int = 0):
    """Seeded row sample: fixed edge positions (first rows, the rows where
    the visible-key count crosses k and the chunk size, the last rows) plus
    uniform rows without replacement, n in total, sorted."""
    edges = {0, m - 2, m - 1, m, m * topk - 2, m * topk - 1, m * topk,
             S - 2, S - 1}
    if chunk > 0:
        edges |= {m * chunk - 1, m * chunk}
    edges = {e for e in edges if 0 <= e < S}
    rng = np.random.default_rng(seed)
    rest = n - len(edges)
    if rest > 0:
        pool = np.setdiff1d(np.arange(S, dtype=np.int64), np.fromiter(edges, np.int64))
        pick = rng.choice(pool, size=min(rest, pool.size), replace=False)
        edges |= set(int(x) for x in pick)
    return np.array(sorted(edges), dtype=np.int64)


def storage_numpy(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a bf16 / fp8 / fp32 tensor as a host numpy array
    (uint16 bits, uint8 codes or float32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


# ------------------------------------------------------------ sparse attention

@dataclass(frozen=True)
class AttnWorkload:
    """Sparse attention over n_sel selected compressed entries per row.

    q [B,S,H,D], k and v [B,T,D] are bf16 with N(0, 1) entries.  Row t (at
    absolute position row_offset + t) sees n = min(T, (pos + 1) // m)
    compressed entries, the indexer's visibility rule; its index list holds
    min(n_sel, n) distinct visible entries followed by -1 padding, the shape
    of the indexer's output.  The pages give no attention dimensions; H = 64
    heads of D = 128 mirror the indexer's.
    """
    name: str
    B: int
    S: int
    T: int
    H: int
    D: int
    n_sel: int
    m: int = 4
    row_offset: int = 0
    scale: float = -1.0     # -1: 1 / sqrt(D)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D)) if self.scale < 0 else self.scale

    def with_(self, **kw) -> "AttnWorkload":
        return replace(self, **kw)


ATTN_WORKLOADS = {
    # the indexer's S = 262,144 shape: the composite step at that length
    "attn-s256k": AttnWorkload("attn-s256k", B=1, S=262144, T=65536, H=64, D=128, n_sel=2048),
    "attn-s64k": AttnWorkload("attn-s64k", B=1, S=65536, T=16384, H=64, D=128, n_sel=2048),
    # the indexer's largest shape, S = 1,048,576
    "attn-s1m": AttnWorkload("attn-s1m", B=1, S=1048576, T=262144, H=64, D=128, n_sel=2048),
    "attn-small": AttnWorkload("attn-small", B=2, S=700, T=175, H=64, D=128, n_sel=100),
    # 64 positions at the end of a 262,144-position context (a decode step)
    "attn-dec64": AttnWorkload("attn-dec64", B=1, S=64, T=65536, H=64, D=128, n_sel=2048,
                               row_offset=262080),
}

_AFFINE_P = 2_147_483_647  # prime: invertible modulo every visible count below it


def make_attn_inputs(aw: AttnWorkload, seed: int = 0, device="cpu"):
    """q [B,S,H,D], k, v [B,T,D] bf16 and idx [B,S,n_sel] int32 on ``device``.

    Row t's list is (P * j + c_t) mod n for j < min(n_sel, n) with P prime
    and c_t uniform in [0, n): distinct entries spread over the whole
    visible range (the order is irrelevant to the attention), then -1.
    """
    B, S, T, H, D, L = aw.B, aw.S, aw.T, aw.H, aw.D, aw.n_sel
    assert T < _AFFINE_P
    q = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=device)
    k = torch.empty((B, T, D), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, T, D), dtype=torch.bfloat16, device=device)
    idx = torch.empty((B, S, L), dtype=torch.int32, device=device)
    j = torch.arange(L, device=device, dtype=torch.int64)
    for b in range(B):
        gq = _generator(device, seed, 10 * b + 5)
        gk = _generator(device, seed, 10 * b + 6)
        gv = _generator(device, seed, 10 * b + 7)
        gi = _generator(device, seed, 10 * b + 8)

        def put_q(r0, r1, x, b=b):
            q[b, r0:r1] = x.to(torch.bfloat16)

        _rows(S, (H, D), "normal", gq, device, put_q)
        k[b] = _draw((T, D), "normal", gk, device).to(torch.bfloat16)
        v[b] = _draw((T, D), "normal", gv, device).to(torch.bfloat16)
        for r0 in range(0, S, _ROW_CHUNK):
            r1 = min(S, r0 + _ROW_CHUNK)
            pos = torch.arange(r0, r1, device=device, dtype=torch.int64) + aw.row_offset
            n = torch.clamp((pos + 1) // aw.m, max=T)
            u = torch.rand((r1 - r0,), generator=gi, device=device, dtype=torch.float64)
            c = torch.minimum((u * n).to(torch.int64), torch.clamp(n - 1, min=0))
            sel = (_AFFINE_P * j[None, :] + c[:, None]) % torch.clamp(n, min=1)[:, None]
            live = j[None, :] < torch.minimum(n, torch.tensor(L, device=device))[:, None]
            idx[b, r0:r1] = torch.where(live, sel, torch.full_like(sel, -1)).to(torch.int32)
    return {"q": q, "k": k, "v": v, "idx": idx}
