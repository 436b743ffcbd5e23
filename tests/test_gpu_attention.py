"""GPU parity of the sparse attention over selected keys (csa_sparse_attention).

Every case runs the HIP kernel through the C ABI and compares rows with the
CPU oracle under the bound that compare_attention derives from the kernel's
arithmetic.  The index lists come from the seeded input module, never from
the HIP indexer, except in the composite test, where the indexer's output on
integer inputs (bit-exact against the oracle, checked there) feeds the
attention.
"""
import numpy as np
import pytest
import torch

from csa_synth import ATTN_WORKLOADS, WORKLOADS, AttnWorkload, make_attn_inputs, make_inputs
from checker import OracleView, attention_reference, compare_attention, compare_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


def _bits(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _check_rows(inp, aw, out, lse, rows_per_b):
    stats = []
    for b, rows in rows_per_b.items():
        rows = np.asarray(rows, np.int64)
        o, l_ref, a, dz = attention_reference(inp, b, rows, aw.softmax_scale)
        r = torch.as_tensor(rows, device=out.device)
        stats.append(compare_attention(_bits(out[b, r]), lse[b, r].cpu().numpy(), o, l_ref, a, dz))
    return stats


def _all_rows(aw):
    return {b: np.arange(aw.S) for b in range(aw.B)}


@pytest.mark.parametrize("H,D", [(32, 64), (32, 128), (64, 64), (64, 128), (128, 64), (128, 128)])
def test_head_and_dim_shapes(csa, H, D):
    """Every built (H, D), two batch entries, 3 full tiles and a ragged
    tail of 4 entries, rows from empty to full lists."""
    aw = AttnWorkload(f"h{H}d{D}", B=2, S=520, T=130, H=H, D=D, n_sel=100)
    print(f"\n[case] {aw}", flush=True)
    inp = make_attn_inputs(aw, seed=1, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], aw.softmax_scale)
    torch.cuda.synchronize()
    stats = _check_rows(inp, aw, out, lse, _all_rows(aw))
    print(f"[attn] {stats}", flush=True)


def test_small_workload_all_rows(csa):
    aw = ATTN_WORKLOADS["attn-small"]
    print(f"\n[case] {aw}", flush=True)
    inp = make_attn_inputs(aw, seed=0, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"])
    torch.cuda.synchronize()
    _check_rows(inp, aw, out, lse, _all_rows(aw))


def test_padding_anywhere_and_out_of_range(csa):
    """-1, other negatives and indices >= T anywhere in a list are skipped;
    whole tiles of padding in the middle of a list are skipped."""
    aw = AttnWorkload("mixed", B=1, S=300, T=200, H=64, D=128, n_sel=130, m=1)
    print(f"\n[case] {aw}", flush=True)
    inp = make_attn_inputs(aw, seed=2, device="cuda")
    idx = inp["idx"].cpu().numpy()
    rng = np.random.default_rng(2)
    for t in range(aw.S):
        row = idx[0, t]
        holes = rng.random(aw.n_sel) < 0.3
        row[holes] = rng.choice([-1, -7, aw.T, aw.T + 5, 2 ** 31 - 1, -2 ** 31], size=holes.sum())
        if t % 7 == 0:
            row[32:96] = -1                    # two empty tiles between full ones
        rng.shuffle(row)
    inp["idx"] = torch.from_numpy(idx).cuda()
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], aw.softmax_scale)
    torch.cuda.synchronize()
    _check_rows(inp, aw, out, lse, _all_rows(aw))


def test_peaked_scores(csa):
    """scale 1 on N(0,1) data: scores ~ N(0, D), the softmax is nearly one-hot
    and the running maximum moves often (rescaling path)."""
    aw = AttnWorkload("peaked", B=1, S=400, T=100, H=64, D=128, n_sel=96, scale=1.0)
    print(f"\n[case] {aw}", flush=True)
    inp = make_attn_inputs(aw, seed=3, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], aw.softmax_scale)
    torch.cuda.synchronize()
    _check_rows(inp, aw, out, lse, _all_rows(aw))


def test_closed_forms(csa):
    """One valid entry: out is that value row, bit for bit (its weight is
    exactly 1).  No valid entry, n_sel = 0 and T = 0: out 0, lse -inf."""
    aw = AttnWorkload("one", B=1, S=64, T=50, H=64, D=128, n_sel=40, m=1)
    inp = make_attn_inputs(aw, seed=4, device="cuda")
    idx = torch.full((1, aw.S, aw.n_sel), -1, dtype=torch.int32)
    rng = np.random.default_rng(4)
    keys = rng.integers(0, aw.T, size=aw.S)
    idx[0, torch.arange(aw.S), torch.as_tensor(rng.integers(0, aw.n_sel, size=aw.S))] = \
        torch.as_tensor(keys, dtype=torch.int32)
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], idx.cuda(), 0.3)
    torch.cuda.synchronize()
    want = inp["v"][0, torch.as_tensor(keys).cuda()][:, None, :].expand(-1, aw.H, -1)
    assert torch.equal(out[0], want)
    assert torch.isfinite(lse).all()

    none = torch.full((1, aw.S, aw.n_sel), -1, dtype=torch.int32, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], none)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))

    empty = torch.empty((1, aw.S, 0), dtype=torch.int32, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], empty)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))

    nokv = torch.empty((1, 0, aw.D), dtype=torch.bfloat16, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], nokv, nokv, inp["idx"])
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))

    # S = 0: nothing to do
    q0 = torch.empty((1, 0, aw.H, aw.D), dtype=torch.bfloat16, device="cuda")
    i0 = torch.empty((1, 0, aw.n_sel), dtype=torch.int32, device="cuda")
    out, lse = csa.sparse_attention(q0, inp["k"], inp["v"], i0)
    assert out.numel() == 0


def test_deterministic_and_lse_optional(csa):
    aw = ATTN_WORKLOADS["attn-small"]
    inp = make_attn_inputs(aw, seed=5, device="cuda")
    a_out, a_lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"])
    b_out, b_lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"])
    c_out, c_lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], want_lse=False)
    torch.cuda.synchronize()
    assert c_lse is None
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse) and torch.equal(a_out, c_out)


def test_full_size_sampled_rows(csa):
    """The S=262,144 shape (T=65,536, H=64, D=128, 2,048 entries per row),
    in the launch configuration the benchmark times; 256 sampled rows,
    including the first rows (short and empty lists), the rows where the
    list first fills (n_vis = 2,048 at position 8,191) and the last."""
    aw = ATTN_WORKLOADS["attn-s256k"]
    print(f"\n[case] {aw}", flush=True)
    inp = make_attn_inputs(aw, seed=0, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    edges = [0, 1, 2, 3, 4, 7, 8190, 8191, 8192, aw.S - 2, aw.S - 1]
    rows = np.unique(np.r_[edges, rng.choice(aw.S, size=256 - len(edges), replace=False)])
    stats = _check_rows(inp, aw, out, lse, {0: rows})
    print(f"[attn] {stats}", flush=True)


def test_s1m_sampled_rows(csa):
    """The largest shape, S=1,048,576 and T=262,144 (43 GB of q, lists and
    output): 128 sampled rows against the oracle."""
    aw = ATTN_WORKLOADS["attn-s1m"]
    print(f"\n[case] {aw}", flush=True)
    inp = make_attn_inputs(aw, seed=0, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    edges = [0, 5, 8191, 8192, aw.S - 1]
    rows = np.unique(np.r_[edges, rng.choice(aw.S, size=128 - len(edges), replace=False)])
    stats = _check_rows(inp, aw, out, lse, {0: rows})
    print(f"[attn] {stats}", flush=True)


def test_composite_after_indexer(csa):
    """The indexer's top-k list feeds the attention: on integer indexer
    inputs the lists equal the oracle's bit for bit, so the attention of
    the oracle's lists is the reference."""
    wl = WORKLOADS["tiny-int"].with_(S=2048, H=64, D=128, k=200)
    print(f"\n[case] {wl}", flush=True)
    ind = make_inputs(wl, seed=0, device="cuda")
    out_idx, out_score = csa.index(ind["q"], ind["w"], ind["k"], wl.m, wl.k)
    aw = AttnWorkload("composite", B=1, S=wl.S, T=wl.n_keys, H=64, D=128, n_sel=wl.k, m=wl.m)
    att = make_attn_inputs(aw, seed=6, device="cuda")
    out, lse = csa.sparse_attention(att["q"], att["k"], att["v"], out_idx)
    torch.cuda.synchronize()
    rows = np.arange(wl.S)
    view = OracleView(ind, wl, 0)
    o_idx, o_score = view.topk(rows, rows, wl.k, wl.m)
    compare_exact(out_idx[0].cpu().numpy(), out_score[0].cpu().numpy(), o_idx, o_score, rows)
    att["idx"] = torch.from_numpy(o_idx[None]).cuda()   # the oracle's lists
    _check_rows(att, aw, out, lse, {0: rows})


# ---------------------------------------------------------------- entry ranges

def _splits(csa, aw, G):
    return csa.attention_plan(csa.make_attn_desc(aw.B, aw.S, aw.T, aw.H, aw.D, aw.n_sel),
                              csa.make_attn_options(G))[0]


@pytest.mark.parametrize("G", [0, 2, 5, 64])
def test_entry_splits_decode(csa, G):
    """64 rows at the end of a 262,144-position context: each row's 2,048
    entries split into ranges (automatic, or 2, 5, 64 of them); every row
    against the oracle."""
    aw = ATTN_WORKLOADS["attn-dec64"]
    got = _splits(csa, aw, G)
    print(f"\n[case] {aw} entry_splits={G} -> {got}", flush=True)
    assert got > 1
    inp = make_attn_inputs(aw, seed=7, device="cuda")
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], entry_splits=G)
    torch.cuda.synchronize()
    stats = _check_rows(inp, aw, out, lse, _all_rows(aw))
    print(f"[attn] {stats}", flush=True)


@pytest.mark.parametrize("H,D", [(32, 64), (64, 128), (128, 64), (128, 128)])
def test_entry_splits_short_lists(csa, H, D):
    """Rows whose lists are shorter than one range (empty ranges, rows with
    no entry at all) and rows whose lists fill several ranges."""
    for off in (0, 1000):
        aw = AttnWorkload(f"split{off}", B=2, S=40, T=3000, H=H, D=D, n_sel=600, row_offset=off)
        print(f"\n[case] {aw} entry_splits=4", flush=True)
        inp = make_attn_inputs(aw, seed=8, device="cuda")
        out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], entry_splits=4)
        torch.cuda.synchronize()
        _check_rows(inp, aw, out, lse, _all_rows(aw))


def test_entry_splits_padding_anywhere(csa):
    aw = AttnWorkload("mixed-split", B=1, S=50, T=900, H=64, D=128, n_sel=700, m=1)
    inp = make_attn_inputs(aw, seed=9, device="cuda")
    idx = inp["idx"].cpu().numpy()
    rng = np.random.default_rng(9)
    for t in range(aw.S):
        row = idx[0, t]
        holes = rng.random(aw.n_sel) < 0.4
        row[holes] = rng.choice([-1, -3, aw.T, aw.T + 9], size=holes.sum())
        if t % 5 == 0:
            row[200:500] = -1              # whole ranges without a valid entry
        rng.shuffle(row)
    inp["idx"] = torch.from_numpy(idx).cuda()
    print(f"\n[case] {aw} entry_splits=3", flush=True)
    out, lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], entry_splits=3)
    torch.cuda.synchronize()
    _check_rows(inp, aw, out, lse, _all_rows(aw))


def test_entry_splits_caller_workspace(csa):
    """A caller workspace with stale content gives the same bits as the
    library-allocated one; repeated calls are bit-identical."""
    aw = ATTN_WORKLOADS["attn-dec64"]
    inp = make_attn_inputs(aw, seed=10, device="cuda")
    a_out, a_lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], entry_splits=0)
    ws = csa.attention_workspace_for(inp["q"], inp["k"], aw.n_sel, entry_splits=0)
    ws.fill_(0x7F)
    b_out, b_lse = csa.sparse_attention(inp["q"], inp["k"], inp["v"], inp["idx"], entry_splits=0,
                                        workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


@pytest.mark.parametrize("G", [1, 3])
def test_equal_weights_exact_mean(csa, G):
    """scale = 0 makes every weight exactly 1 (bf16 of 2^0): the output is
    the mean of the selected value rows.  Checked against the oracle (the
    exact mean, within one bf16 step) and, since with integer values the
    sum and the weight count are exact in fp32, bit for bit against
    bf16(f32(sum v) * f32(1 / n)), with and without entry ranges; lse =
    log(n)."""
    aw = AttnWorkload("mean", B=2, S=96, T=300, H=64, D=128, n_sel=200, m=1)
    inp = make_attn_inputs(aw, seed=13, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(13)
    v = torch.randint(-3, 4, (aw.B, aw.T, aw.D), generator=g).to(torch.bfloat16).cuda()
    out, lse = csa.sparse_attention(inp["q"], inp["k"], v, inp["idx"], 0.0, entry_splits=G)
    torch.cuda.synchronize()
    idx = inp["idx"].cpu().numpy()
    vf = v.float().cpu().numpy()
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    import oracle
    from csa_synth import storage_numpy
    for b in range(aw.B):
        # the oracle (fp64) at scale 0: the exact mean of the selected value
        # rows; the kernel's output is that mean rounded to bf16 (through an
        # fp32 product), so within one bf16 step of it
        o, o_lse, _ = oracle.sparse_attention(storage_numpy(inp["q"][b]), storage_numpy(inp["k"][b]),
                                              storage_numpy(v[b]), idx[b], 0.0)
        assert np.all(np.abs(got[b] - o) <= 2.0 ** -8 * np.abs(o)), b
        assert np.array_equal(np.isneginf(got_lse[b]), np.isneginf(o_lse))
        fin = np.isfinite(o_lse)
        np.testing.assert_allclose(got_lse[b][fin], o_lse[fin], rtol=1e-6)
        for t in range(aw.S):
            sel = idx[b, t][(idx[b, t] >= 0) & (idx[b, t] < aw.T)]
            n = len(sel)
            if n == 0:
                assert np.all(got[b, t] == 0) and np.all(np.isneginf(got_lse[b, t]))
                continue
            s = vf[b, sel].sum(axis=0).astype(np.float32)          # exact: small integers
            want = torch.from_numpy(s * (np.float32(1) / np.float32(n))).to(torch.bfloat16)
            assert np.array_equal(got[b, t], np.broadcast_to(want.float().numpy(), (aw.H, aw.D))), (b, t)
            np.testing.assert_allclose(got_lse[b, t], np.log(n), rtol=1e-6)
