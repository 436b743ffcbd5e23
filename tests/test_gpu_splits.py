"""GPU parity of the key-range path.

Short query blocks at the end of a long context (a decode step, the last
rows of a chunked prefill) leave most compute units idle when only query
blocks are spread over the device; the library then splits each block's
visible keys into ranges scored by separate workgroups and merges the
ranges' top-k lists.  The result is defined to be the same as without the
split: every row is checked against the oracle (bit-exact on integer
inputs), and outputs are bit-identical across split counts.
"""
import numpy as np
import pytest
import torch

from csa_synth import WORKLOADS, Workload, make_inputs
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
                    k_scale=inp.get("k_scale"), row_offset=wl.row_offset, **kw)
    torch.cuda.synchronize()
    return out


def _splits(csa, wl, key_splits=0):
    info = csa.plan_query(csa.make_desc(wl.B, wl.S, wl.n_keys, wl.H, wl.D), wl.m, wl.k,
                          csa.make_options(row_offset=wl.row_offset, key_splits=key_splits))
    return info.key_splits


def _check_all_rows(inp, wl, out_idx, out_score, exact):
    rows = np.arange(wl.S)
    t_rows = rows + wl.row_offset
    stats = []
    for b in range(wl.B):
        view = OracleView(inp, wl, b)
        o_idx, o_score = view.topk(rows, t_rows, wl.k, wl.m)
        g_idx = out_idx[b].cpu().numpy()
        g_score = out_score[b].cpu().numpy()
        if exact:
            compare_exact(g_idx, g_score, o_idx, o_score, t_rows)
        else:
            stats.append(compare_tolerant(g_idx, g_score, o_idx, o_score,
                                          lambda pr, pk: view.score(rows, pr, pk), t_rows,
                                          wl.n_keys, wl.m))
    return stats


def test_dec64_int_exact(csa):
    wl = WORKLOADS["dec64-int"]
    G = _splits(csa, wl)
    print(f"\n[case] {wl} key_splits={G}", flush=True)
    assert G > 1
    inp = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = _run(csa, inp, wl)
    _check_all_rows(inp, wl, out_idx, out_score, exact=True)


def test_dec64_gauss_all_rows(csa):
    wl = WORKLOADS["dec64"]
    print(f"\n[case] {wl} key_splits={_splits(csa, wl)}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = _run(csa, inp, wl)
    stats = _check_all_rows(inp, wl, out_idx, out_score, exact=False)
    print(f"[splits] {stats}", flush=True)
    assert min(s["recall"] for s in stats) > 0.999


def test_split_counts_bit_identical(csa):
    """1 (no split), a few uneven ranges, the automatic count, and ranges of
    256 keys (smaller than k, so every range returns all its keys); and the
    range kernel with 64-key and 128-key staged tiles."""
    wl = WORKLOADS["dec64"]
    inp = make_inputs(wl, seed=1, device="cuda")
    ref = None
    for G in (1, 2, 7, 0, 256):
        print(f"\n[case] {wl.name} key_splits={G} -> {_splits(csa, wl, G)}", flush=True)
        got = _run(csa, inp, wl, key_splits=G)
        if ref is None:
            ref = got
            continue
        assert torch.equal(got[0], ref[0]), f"indices differ at key_splits={G}"
        assert torch.equal(got[1], ref[1]), f"scores differ at key_splits={G}"
    # the range kernel's two staged key tiles (128 is its default here)
    for G in (0, 7):
        print(f"\n[case] {wl.name} key_splits={G} key_tile=64", flush=True)
        got = _run(csa, inp, wl, key_splits=G, key_tile=64)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), G


def test_dec32x4_batch(csa):
    wl = WORKLOADS["dec32x4"]
    G = _splits(csa, wl)
    print(f"\n[case] {wl} key_splits={G}", flush=True)
    assert G > 1
    inp = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = _run(csa, inp, wl)
    stats = _check_all_rows(inp, wl, out_idx, out_score, exact=False)
    assert min(s["recall"] for s in stats) > 0.999


@pytest.mark.parametrize("wl,G", [
    # 8 ranges of 64 keys from the first position on: the early blocks see
    # fewer keys than the later ranges start at, so many units are empty
    (Workload("early", B=1, S=2048, m=4, H=64, D=128, k=100, T=4000, dist="int"), 8),
    # k above every row's visible count (about 500): padding from every range
    (Workload("pad", B=1, S=16, m=4, H=64, D=128, k=2048, T=1000, row_offset=2000,
              dist="int"), 4),
    # no keys at all
    (Workload("nokeys", B=1, S=20, m=4, H=64, D=128, k=8, T=0, dist="int"), 3),
    # 16 positions per wave (H = 4, d = 32), two batch entries
    (Workload("h4", B=2, S=40, m=4, H=4, D=32, k=64, T=3000, row_offset=11000,
              dist="int"), 6),
    # fp8 operands with unit scales
    (Workload("fp8", B=1, S=16, m=4, H=64, D=128, k=256, T=5000, row_offset=19990,
              dist="int", dtype="e4m3fn"), 5),
], ids=lambda x: x.name if isinstance(x, Workload) else str(x))
def test_split_edge_cases_exact(csa, wl, G):
    got = _splits(csa, wl, G)
    print(f"\n[case] {wl} key_splits={G} -> {got}", flush=True)
    assert got == (G if wl.n_keys > 0 else 1)
    inp = make_inputs(wl, seed=3, device="cuda")
    out_idx, out_score = _run(csa, inp, wl, key_splits=G)
    if wl.n_keys == 0:
        assert torch.all(out_idx == -1) and torch.all(torch.isneginf(out_score))
        return
    _check_all_rows(inp, wl, out_idx, out_score, exact=True)


def test_split_caller_workspace(csa):
    wl = WORKLOADS["dec64-int"]
    inp = make_inputs(wl, seed=4, device="cuda")
    a = _run(csa, inp, wl)
    ws = csa.workspace_for(inp["q"], inp["k"], wl.m, wl.k, row_offset=wl.row_offset)
    ws.fill_(0x5A)  # stale content must not matter
    b = _run(csa, inp, wl, workspace=ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
