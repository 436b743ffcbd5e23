"""GPU parity at the benchmark sizes (sampled rows) and structural properties.

The full-size calls run in the same configuration bench.py times (default
chunk, one call over the whole workload); the oracle checks a seeded
256-row sample of each.  Properties that hold at any size (chunk-size
invariance, determinism, row_offset slicing, workspace ownership) are
checked on every row.
"""
import numpy as np
import pytest
import torch

from csa_synth import (CHUNK_SWEEP, KEY_TILE_SWEEP, RANGE_SWEEP, TOPK_SWEEP, WORKLOADS, Workload,
                       make_inputs, sample_rows)
from checker import OracleView, compare_exact, compare_tolerant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


def _run(csa, inp, wl, **kw):
    out = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, q_scale=inp.get("q_scale"),
                    k_scale=inp.get("k_scale"), **kw)
    torch.cuda.synchronize()
    return out


def _sample_check(inp, wl, out_idx, out_score, rows, exact):
    view = OracleView(inp, wl, 0)
    o_idx, o_score = view.topk(rows, rows, wl.k, wl.m)
    rt = torch.as_tensor(rows, device="cuda")
    g_idx = out_idx[0].index_select(0, rt).cpu().numpy()
    g_score = out_score[0].index_select(0, rt).cpu().numpy()
    if exact:
        compare_exact(g_idx, g_score, o_idx, o_score, rows)
        return None
    return compare_tolerant(g_idx, g_score, o_idx, o_score,
                            lambda pr, pk: view.score(rows, pr, pk), rows, wl.n_keys, wl.m)


def test_s64k_chunk_sweep_bit_identical_and_sampled(csa):
    wl = WORKLOADS["s64k"]
    print(f"\n[case] {wl} chunks {CHUNK_SWEEP}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    ref_idx, ref_score = _run(csa, inp, wl, chunk_keys=CHUNK_SWEEP[0])
    for c in CHUNK_SWEEP[1:]:
        print(f"[case] chunk {c}", flush=True)
        idx, score = _run(csa, inp, wl, chunk_keys=c)
        assert torch.equal(idx, ref_idx), f"indices differ at chunk {c}"
        assert torch.equal(score, ref_score), f"scores differ at chunk {c}"
        del idx, score
    rows = sample_rows(wl.S, wl.m, wl.k, n=256, chunk=CHUNK_SWEEP[0])
    stats = _sample_check(inp, wl, ref_idx, ref_score, rows, exact=False)
    print(f"[sweep] chunks {CHUNK_SWEEP} k={wl.k} {stats}", flush=True)
    assert stats["recall"] > 0.999


def test_s64k_key_tile_and_range_sweeps_bit_identical(csa):
    """The staged key-tile sweep (32 ... 256 keys) and the key-range sweep
    (ranges of 1,024 ... 16,384 keys, each range's exact top-k merged) of
    the S=65,536 workload: every cell bit-identical to the default call,
    which matches the oracle on 256 sampled rows."""
    wl = WORKLOADS["s64k"]
    print(f"\n[case] {wl} key tiles {KEY_TILE_SWEEP} ranges {RANGE_SWEEP}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    ref_idx, ref_score = _run(csa, inp, wl)
    for kt in KEY_TILE_SWEEP:
        print(f"[case] key_tile {kt}", flush=True)
        idx, score = _run(csa, inp, wl, key_tile=kt)
        assert torch.equal(idx, ref_idx), f"indices differ at key tile {kt}"
        assert torch.equal(score, ref_score), f"scores differ at key tile {kt}"
        del idx, score
    for r in RANGE_SWEEP:
        G = wl.n_keys // r
        print(f"[case] {G} key ranges of {r} keys", flush=True)
        idx, score = _run(csa, inp, wl, key_splits=G)
        assert torch.equal(idx, ref_idx), f"indices differ with ranges of {r} keys"
        assert torch.equal(score, ref_score), f"scores differ with ranges of {r} keys"
        del idx, score
    rows = sample_rows(wl.S, wl.m, wl.k, n=256)
    stats = _sample_check(inp, wl, ref_idx, ref_score, rows, exact=False)
    print(f"[sweep] key tiles and ranges k={wl.k} {stats}", flush=True)
    assert stats["recall"] > 0.999


@pytest.mark.parametrize("k", [k for k in TOPK_SWEEP if k != WORKLOADS["s64k"].k])
def test_s64k_topk_sweep_sampled(csa, k):
    """The top-k sweep cells of the S=65,536 workload (k = 2048 is the
    chunk-sweep test above): sampled rows against the oracle."""
    wl = WORKLOADS["s64k"].with_(k=k)
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = _run(csa, inp, wl)
    rows = sample_rows(wl.S, wl.m, wl.k, n=256)
    stats = _sample_check(inp, wl, out_idx, out_score, rows, exact=False)
    print(f"[sweep] k={k} {stats}", flush=True)
    assert stats["recall"] > 0.999


@pytest.mark.parametrize("name", ["s256k", "s256k-int"])
def test_s256k_sampled(csa, name):
    wl = WORKLOADS[name]
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = _run(csa, inp, wl)
    rows = sample_rows(wl.S, wl.m, wl.k, n=256)
    print(_sample_check(inp, wl, out_idx, out_score, rows, exact=wl.dist == "int"))


@pytest.mark.parametrize("name", ["s1m-fp8-int", "s1m-fp8"])
def test_s1m_fp8_sampled(csa, name):
    wl = WORKLOADS[name]
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = _run(csa, inp, wl)
    rows = sample_rows(wl.S, wl.m, wl.k, n=256)
    print(_sample_check(inp, wl, out_idx, out_score, rows, exact=wl.dist == "int"))


def test_deterministic(csa):
    wl = WORKLOADS["s16k"]
    print(f"\n[case] determinism {wl}", flush=True)
    inp = make_inputs(wl, seed=1, device="cuda")
    a = _run(csa, inp, wl)
    b = _run(csa, inp, wl)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_row_offset_suffix_equals_full_run(csa):
    wl = Workload("offset", B=1, S=6000, m=4, H=64, D=128, k=300)
    print(f"\n[case] row_offset {wl}", flush=True)
    inp = make_inputs(wl, seed=2, device="cuda")
    full_idx, full_score = _run(csa, inp, wl)
    for start in (1, 2500, 5999):
        part = {"q": inp["q"][:, start:].contiguous(), "w": inp["w"][:, start:].contiguous(),
                "k": inp["k"]}
        sub = wl.with_(S=wl.S - start, T=wl.n_keys)
        idx, score = _run(csa, part, sub, row_offset=start)
        assert torch.equal(idx, full_idx[:, start:]), start
        assert torch.equal(score, full_score[:, start:]), start


def test_caller_workspace_matches_library_workspace(csa):
    wl = Workload("ws", B=2, S=3000, m=4, H=64, D=128, k=256, dist="int")
    print(f"\n[case] workspace {wl}", flush=True)
    inp = make_inputs(wl, seed=3, device="cuda")
    a = _run(csa, inp, wl)
    ws = csa.workspace_for(inp["q"], inp["k"], wl.m, wl.k)
    ws.fill_(0xAB)  # stale content must not matter
    b = _run(csa, inp, wl, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_degenerate_shapes(csa):
    # no keys at all: every row is padding
    wl = Workload("nokeys", B=1, S=50, m=4, H=64, D=128, k=5, T=0)
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=4, device="cuda")
    idx, score = _run(csa, inp, wl)
    assert torch.all(idx == -1) and torch.all(torch.isneginf(score))
    # a single position, k = 1
    wl = Workload("one", B=1, S=1, m=1, H=4, D=32, k=1, dist="int")
    inp = make_inputs(wl, seed=5, device="cuda")
    idx, score = _run(csa, inp, wl)
    view = OracleView(inp, wl, 0)
    o_idx, o_score = view.topk(np.array([0]), np.array([0]), wl.k, wl.m)
    compare_exact(idx[0].cpu().numpy(), score[0].cpu().numpy(), o_idx, o_score)


def test_all_scores_tied(csa):
    """q = 0: every visible key scores exactly 0, so each row must return the
    lowest visible key indices in ascending order (ties to the lower index)."""
    wl = Workload("ties", B=1, S=5000, m=4, H=64, D=128, k=200, dist="int")
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=6, device="cuda")
    inp["q"].zero_()
    for chunk in (64, 0):
        idx, score = _run(csa, inp, wl, chunk_keys=chunk)
        t = torch.arange(wl.S, device="cuda")
        n = torch.clamp((t + 1) // wl.m, max=wl.n_keys)
        slot = torch.arange(wl.k, device="cuda")
        want = torch.where(slot[None, :] < n[:, None], slot[None, :], torch.full_like(slot, -1)[None, :])
        assert torch.equal(idx[0], want.to(torch.int32))
        assert torch.all(score[0][want >= 0] == 0)
