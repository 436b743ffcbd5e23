"""GPU checks of the entry points' documented properties.

* csa_index (default options) equals csa_index_ex.
* With a caller workspace a call only enqueues kernels on the stream, so it
  can be captured into a HIP graph; every replay must match the eager call
  (the graph holds no memset node, the library allocates nothing).
* The library keeps no state between calls: two streams running calls with
  their own workspaces at the same time produce the eager results.
"""
import ctypes

import pytest
import torch

from csa_synth import Workload, make_inputs

pytestmark = pytest.mark.gpu

WL = Workload("api", B=2, S=1500, m=4, H=64, D=128, k=128, T=-1)


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


@pytest.fixture(scope="module")
def inputs():
    return make_inputs(WL, seed=11, device="cuda")


def _eager(csa, inp, **kw):
    out = csa.index(inp["q"], inp["w"], inp["k"], WL.m, WL.k, **kw)
    torch.cuda.synchronize()
    return out


def test_csa_index_default_entry_point(csa, inputs):
    from streaming_top_selection_csa_amd import binding as B
    ref_idx, ref_score = _eager(csa, inputs)
    q, w, k = inputs["q"], inputs["w"], inputs["k"]
    out_idx = torch.empty_like(ref_idx)
    out_score = torch.empty_like(ref_score)
    desc = B.make_desc(WL.B, WL.S, WL.n_keys, WL.H, WL.D)
    stream = torch.cuda.current_stream()
    rc = B.load_library().csa_index(q.data_ptr(), w.data_ptr(), k.data_ptr(), ctypes.byref(desc),
                                    WL.m, WL.k, out_idx.data_ptr(), out_score.data_ptr(),
                                    ctypes.c_void_p(stream.cuda_stream))
    assert rc == B.CSA_OK
    torch.cuda.synchronize()
    assert torch.equal(out_idx, ref_idx) and torch.equal(out_score, ref_score)


def test_graph_capture_replays(csa, inputs):
    ref_idx, ref_score = _eager(csa, inputs)
    ws = csa.workspace_for(inputs["q"], inputs["k"], WL.m, WL.k)
    out_idx = torch.empty_like(ref_idx)
    out_score = torch.empty_like(ref_score)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            csa.index(inputs["q"], inputs["w"], inputs["k"], WL.m, WL.k, out_idx=out_idx,
                      out_score=out_score, workspace=ws, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        out_idx.fill_(7)
        out_score.fill_(7.0)
        ws.fill_(rep)  # the workspace's stale content never matters
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_idx, ref_idx), f"replay {rep}: indices"
        assert torch.equal(out_score, ref_score), f"replay {rep}: scores"
        _eager(csa, inputs)  # eager work between the replays


def test_concurrent_streams(csa, inputs):
    ref_idx, ref_score = _eager(csa, inputs)
    streams = [torch.cuda.Stream() for _ in range(2)]
    wss = [csa.workspace_for(inputs["q"], inputs["k"], WL.m, WL.k) for _ in streams]
    outs = [(torch.empty_like(ref_idx), torch.empty_like(ref_score)) for _ in streams]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for st, ws, (oi, os_) in zip(streams, wss, outs):
            with torch.cuda.stream(st):
                csa.index(inputs["q"], inputs["w"], inputs["k"], WL.m, WL.k, out_idx=oi,
                          out_score=os_, workspace=ws, stream=st)
    torch.cuda.synchronize()
    for oi, os_ in outs:
        assert torch.equal(oi, ref_idx) and torch.equal(os_, ref_score)


def test_attention_graph_capture_and_streams(csa):
    """csa_sparse_attention allocates nothing, and with a caller workspace
    the range-split form only enqueues kernels too: both can be captured
    into a HIP graph, and every replay (with eager work between) matches
    the eager call.  Two streams running split calls with their own
    workspaces at the same time also match."""
    from csa_synth import ATTN_WORKLOADS, make_attn_inputs
    aw = ATTN_WORKLOADS["attn-dec64"]
    inp = make_attn_inputs(aw, seed=12, device="cuda")
    args = (inp["q"], inp["k"], inp["v"], inp["idx"])
    for G in (1, 0):
        ref_out, ref_lse = csa.sparse_attention(*args, entry_splits=G)
        torch.cuda.synchronize()
        ws = csa.attention_workspace_for(inp["q"], inp["k"], aw.n_sel, entry_splits=G)
        out = torch.empty_like(ref_out)
        lse = torch.empty_like(ref_lse)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                csa.sparse_attention(*args, out=out, lse=lse, entry_splits=G, workspace=ws,
                                     stream=side)
        torch.cuda.synchronize()
        for rep in range(3):
            out.fill_(3)
            lse.fill_(3.0)
            ws.fill_(rep + 1)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"G={G} replay {rep}"
            csa.sparse_attention(*args, entry_splits=G)  # eager work between the replays

    ref_out, ref_lse = csa.sparse_attention(*args, entry_splits=0)
    streams = [torch.cuda.Stream() for _ in range(2)]
    wss = [csa.attention_workspace_for(inp["q"], inp["k"], aw.n_sel, 0) for _ in streams]
    outs = [(torch.empty_like(ref_out), torch.empty_like(ref_lse)) for _ in streams]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for st, ws, (o, l) in zip(streams, wss, outs):
            with torch.cuda.stream(st):
                csa.sparse_attention(*args, out=o, lse=l, entry_splits=0, workspace=ws, stream=st)
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_out) and torch.equal(l, ref_lse)
