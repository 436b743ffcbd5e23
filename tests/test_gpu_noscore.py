"""Calls without a score output (out_score = NULL) through the C ABI.

The indices must be bit-identical to the call with scores, and exact
against the oracle on integer-valued inputs: for rows the scoring kernel
sorts itself (next_pow2(k) <= 2048, no key ranges) and for rows sorted by
the separate pass (key ranges, larger k), whose scores then live in the
workspace.
"""
import numpy as np
import pytest
import torch

from csa_synth import WORKLOADS, Workload, make_inputs, sample_rows
from checker import OracleView, compare_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


def _both(csa, inp, wl, **kw):
    idx, score = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, q_scale=inp.get("q_scale"),
                           k_scale=inp.get("k_scale"), row_offset=wl.row_offset, **kw)
    idx2, none = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, q_scale=inp.get("q_scale"),
                           k_scale=inp.get("k_scale"), row_offset=wl.row_offset, want_score=False,
                           **kw)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(idx, idx2)
    return idx, score


CASES = [
    # (B, S, m, H, D, k, T, row_offset, key_splits)
    (1, 3000, 4, 64, 128, 512, -1, 0, 0),      # sorted in the kernel, 8 keys per lane
    (1, 3000, 4, 64, 128, 2048, -1, 0, 0),     # sorted in the kernel, 32 keys per lane
    (2, 700, 2, 8, 64, 100, -1, 0, 0),         # several positions per wave
    (1, 64, 4, 64, 128, 512, 4096, 16320, 0),  # key ranges, few rows: the merge kernel sorts
    (1, 3000, 4, 64, 128, 512, -1, 0, 4),      # key ranges, many rows: separate sort, scores in workspace
    (1, 900, 1, 16, 32, 3000, -1, 0, 0),       # k > 2048: separate sort, scores in workspace
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dS%dm%dH%dD%dk%dT%do%dG%d" % c)
def test_no_score_integer_exact(csa, case):
    B, S, m, H, D, k, T, off, G = case
    wl = Workload("noscore", B=B, S=S, m=m, H=H, D=D, k=k, dist="int", T=T, row_offset=off)
    print(f"\n[case] {wl} key_splits={G}", flush=True)
    inp = make_inputs(wl, seed=S + k, device="cuda")
    idx, score = _both(csa, inp, wl, key_splits=G)
    for b in range(B):
        view = OracleView(inp, wl, b)
        r = np.arange(S, dtype=np.int64)
        o_idx, o_score = view.topk(r, r + off, k, m)
        compare_exact(idx[b].cpu().numpy(), score[b].cpu().numpy(), o_idx, o_score, r + off)


@pytest.mark.parametrize("name", ["s256k-int", "s1m-fp8-int"])
def test_no_score_full_size_sample(csa, name):
    """The benchmark shapes: indices identical with and without scores, and
    exact against the oracle on 256 sampled rows."""
    wl = WORKLOADS[name]
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    idx, score = _both(csa, inp, wl)
    view = OracleView(inp, wl, 0)
    rows = sample_rows(wl.S, wl.m, wl.k)
    o_idx, o_score = view.topk(rows, rows, wl.k, wl.m)
    rt = torch.as_tensor(rows, device="cuda")
    compare_exact(idx[0].index_select(0, rt).cpu().numpy(),
                  score[0].index_select(0, rt).cpu().numpy(), o_idx, o_score, rows)
