"""csa_index_static (no allocation: the library's fixed device scratch)
through the C ABI, against csa_index_ex on the same inputs.

Two calls in a row on one GPU, the second smaller, so the second runs on
scratch the first left behind.  Results must be bit-identical to
csa_index_ex (the partition size it may pick changes no result); the
integer-valued calls are also exact against the oracle.
"""
import numpy as np
import pytest
import torch

from csa_synth import WORKLOADS, Workload, make_inputs
from checker import OracleView, compare_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


def _pair(csa, inp, wl, **kw):
    args = dict(q_scale=inp.get("q_scale"), k_scale=inp.get("k_scale"), row_offset=wl.row_offset)
    args.update(kw)
    ref_idx, ref_score = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, **args)
    idx, score = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, static_scratch=True, **args)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    assert torch.equal(score, ref_score)
    return idx, score


def _exact(inp, wl, idx, score):
    view = OracleView(inp, wl, 0)
    rows = np.arange(wl.S, dtype=np.int64)
    o_idx, o_score = view.topk(rows, rows + wl.row_offset, wl.k, wl.m)
    compare_exact(idx[0].cpu().numpy(), score[0].cpu().numpy(), o_idx, o_score,
                  rows + wl.row_offset)


def test_static_scratch_two_calls(csa):
    # a large call whose default candidate logs (168 MB) exceed the scratch:
    # the partition size is lowered until they fit
    big = WORKLOADS["s64k"]
    print(f"\n[case] {big} static scratch", flush=True)
    d = csa.make_desc(big.B, big.S, big.n_keys, big.H, big.D)
    assert csa.workspace_bytes(d, big.m, big.k, csa.make_options(num_cus=256)) > \
        csa.STATIC_SCRATCH_BYTES
    inp = make_inputs(big, seed=0, device="cuda")
    _pair(csa, inp, big)
    del inp
    # then a smaller, integer-valued call on the scratch the first one left
    small = Workload("small", B=1, S=3000, m=4, H=64, D=128, k=512, dist="int")
    print(f"[case] {small} static scratch", flush=True)
    inp = make_inputs(small, seed=1, device="cuda")
    idx, score = _pair(csa, inp, small)
    _exact(inp, small, idx, score)


def test_static_scratch_key_ranges_and_no_score(csa):
    """A decode-shaped call (key ranges, merge and sort passes), with and
    without scores, twice in a row with a smaller second call."""
    wl = WORKLOADS["dec64-int"]
    print(f"\n[case] {wl} static scratch", flush=True)
    inp = make_inputs(wl, seed=0, device="cuda")
    idx, score = _pair(csa, inp, wl)
    idx2, none = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, row_offset=wl.row_offset,
                           static_scratch=True, want_score=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(idx2, idx)
    _exact(inp, wl, idx, score)
    small = wl.with_(S=16, row_offset=4 * 65536 - 16)
    print(f"[case] {small} static scratch", flush=True)
    inp = make_inputs(small, seed=2, device="cuda")
    idx, score = _pair(csa, inp, small)
    _exact(inp, small, idx, score)
