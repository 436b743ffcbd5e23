"""The grouped (approximate) indexer, csa_index_grouped, through the C ABI.

Integer-valued inputs with full groups of 8 or 16 positions keep every
pooled score exact in fp32, so the GPU must match the grouped oracle
(oracle/csa_group_oracle.c) bit for bit on every row.  With a candidate
count covering every visible key the grouped result must equal csa_index
bit for bit (every member then scores all of its keys), on gaussian
inputs too.
"""
import numpy as np
import pytest
import torch

from csa_synth import Workload, make_inputs, storage_numpy
from checker import compare_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


CASES = [
    # (B, S, T, m, k, g, C, row_offset)
    (1, 2048, 512, 4, 64, 8, 64, 0),
    (1, 2048, 512, 4, 64, 8, 200, 0),
    (2, 1024, 256, 4, 100, 16, 150, 0),
    (1, 1536, 700, 2, 32, 8, 2000, 0),       # many candidates (separate scan sort)
    (1, 512, 1024, 4, 128, 16, 300, 3000),   # a shard deep in a longer sequence
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dS%dT%dm%dk%dg%dC%do%d" % c)
def test_grouped_integer_exact_vs_grouped_oracle(csa, case):
    import oracle
    B, S, T, m, k, g, C, off = case
    wl = Workload("grouped", B=B, S=S, m=m, H=64, D=128, k=k, dist="int", T=T, row_offset=off)
    print(f"\n[case] {wl} group={g} candidates={C}", flush=True)
    inp = make_inputs(wl, seed=S + g, device="cuda")
    idx, score = csa.index_grouped(inp["q"], inp["w"], inp["k"], m, k, g, C, row_offset=off)
    idx2, none = csa.index_grouped(inp["q"], inp["w"], inp["k"], m, k, g, C, row_offset=off,
                                   want_score=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(idx, idx2)
    rows = np.arange(S, dtype=np.int64)
    for b in range(B):
        o_idx, o_score = oracle.grouped_rows(storage_numpy(inp["q"][b]), inp["w"][b].cpu().numpy(),
                                             storage_numpy(inp["k"][b]), rows, m, k, g, C,
                                             row_offset=off)
        compare_exact(idx[b].cpu().numpy(), score[b].cpu().numpy(), o_idx, o_score, rows + off)


@pytest.mark.parametrize("dist", ["int", "gauss"])
def test_grouped_with_all_keys_as_candidates_equals_exact(csa, dist):
    wl = Workload("grouped-all", B=1, S=4096, m=4, H=64, D=128, k=256, dist=dist, T=1024)
    print(f"\n[case] {wl} group=32 candidates=8192", flush=True)
    inp = make_inputs(wl, seed=7, device="cuda")
    gi, gs = csa.index_grouped(inp["q"], inp["w"], inp["k"], wl.m, wl.k, 32, 8192)
    ei, es = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k)
    torch.cuda.synchronize()
    assert torch.equal(gi, ei)
    assert torch.equal(gs, es)


def test_grouped_validation(csa):
    wl = Workload("grouped-bad", B=1, S=64, m=4, H=32, D=128, k=16, dist="int")
    inp = make_inputs(wl, seed=1, device="cuda")
    with pytest.raises(csa.CsaError) as e:
        csa.index_grouped(inp["q"], inp["w"], inp["k"], 4, 16, 8)
    assert e.value.status == -2        # H = 32: unsupported
    wl = wl.with_(H=64)
    inp = make_inputs(wl, seed=1, device="cuda")
    for g, C in ((12, 0), (8, 8), (8, 9000)):   # g not a multiple of 8; C < k; C too large
        with pytest.raises(csa.CsaError) as e:
            csa.index_grouped(inp["q"], inp["w"], inp["k"], 4, 16, g, C)
        assert e.value.status == -1
