"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer-valued inputs must match bit for bit (indices and scores); gaussian
inputs must meet the tolerance rule in tests/checker.py.
"""
import numpy as np
import pytest
import torch

from csa_synth import CHUNK_SWEEP, KEY_TILE_SWEEP, WORKLOADS, Workload, make_inputs, sample_rows
from checker import OracleView, compare_exact, compare_tolerant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_top_selection_csa_amd as lib
    lib.load_library()
    return lib


def _run(csa, inp, wl, chunk=0, row_offset=0, key_tile=0):
    out_idx, out_score = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k,
                                   q_scale=inp.get("q_scale"), k_scale=inp.get("k_scale"),
                                   chunk_keys=chunk, row_offset=row_offset, key_tile=key_tile)
    torch.cuda.synchronize()
    return out_idx, out_score


def _check(csa, wl, seed=0, rows=None, chunk=0, exact=None, b_list=None, key_tile=0):
    print(f"\n[case] {wl} seed={seed} chunk={chunk} key_tile={key_tile}", flush=True)
    inp = make_inputs(wl, seed=seed, device="cuda")
    out_idx, out_score = _run(csa, inp, wl, chunk=chunk, key_tile=key_tile)
    exact = (wl.dist == "int") if exact is None else exact
    stats = []
    for b in (b_list if b_list is not None else range(wl.B)):
        view = OracleView(inp, wl, b)
        r = np.arange(wl.S, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
        o_idx, o_score = view.topk(r, r, wl.k, wl.m)
        g_idx = out_idx[b].index_select(0, torch.as_tensor(r, device="cuda")).cpu().numpy()
        g_score = out_score[b].index_select(0, torch.as_tensor(r, device="cuda")).cpu().numpy()
        if exact:
            compare_exact(g_idx, g_score, o_idx, o_score, r)
        else:
            stats.append(compare_tolerant(g_idx, g_score, o_idx, o_score,
                                          lambda pr, pk: view.score(r, pr, pk),
                                          r, wl.n_keys, wl.m))
    return out_idx, out_score, stats


def test_tiny_int_all_rows(csa):
    _check(csa, WORKLOADS["tiny-int"])


SMALL_EXACT = [
    # (B, S, m, H, D, k, T)  integer inputs, every row checked
    (1, 200, 4, 64, 128, 16, -1),
    (1, 1000, 4, 64, 128, 100, -1),
    (2, 777, 3, 64, 128, 37, -1),
    (1, 513, 1, 32, 64, 64, -1),
    (1, 300, 2, 16, 128, 200, -1),
    (1, 2049, 4, 8, 32, 512, -1),
    (1, 257, 2, 4, 64, 1, -1),
    (1, 129, 1, 2, 32, 130, -1),
    (1, 100, 1, 1, 32, 7, -1),
    (1, 90, 1, 64, 128, 5, 40),      # T smaller than S/m: every late row sees all keys
    (1, 3000, 4, 64, 128, 2048, -1),  # k larger than most visible sets
    (1, 14000, 4, 64, 128, 3000, -1),  # rows wider than 2048: workgroup row sort in LDS
    (1, 21000, 4, 64, 128, 5000, -1),  # same, 8192-key rows
]


@pytest.mark.parametrize("shape", SMALL_EXACT, ids=lambda s: "B%dS%dm%dH%dD%dk%dT%d" % s)
def test_small_integer_exact(csa, shape):
    B, S, m, H, D, k, T = shape
    _check(csa, Workload("small", B=B, S=S, m=m, H=H, D=D, k=k, dist="int", T=T), seed=S)


@pytest.mark.parametrize("key_tile", KEY_TILE_SWEEP)
@pytest.mark.parametrize("shape", [(1, 3001, 4, 100, 750), (2, 999, 3, 2048, -1),
                                   (1, 1203, 1, 37, 1203)], ids=lambda s: "B%dS%dm%dk%dT%d" % s)
def test_key_tiles_integer_exact(csa, shape, key_tile):
    """Every staged key-tile size, on integer inputs whose key counts are no
    multiple of any tile (ragged last tiles), every row exact."""
    B, S, m, k, T = shape
    _check(csa, Workload("tiles", B=B, S=S, m=m, H=64, D=128, k=k, dist="int", T=T), seed=S + k,
           key_tile=key_tile)


@pytest.mark.parametrize("chunk", [64, 192, 1024])
def test_small_integer_chunks(csa, chunk):
    """A small merge interval forces many merges per row."""
    wl = Workload("small", B=1, S=4000, m=4, H=64, D=128, k=100, dist="int")
    _check(csa, wl, seed=7, chunk=chunk)


def test_gauss_all_rows(csa):
    wl = Workload("gauss", B=1, S=4096, m=4, H=64, D=128, k=256)
    _, _, stats = _check(csa, wl, seed=3)
    print(stats)


def test_fp8_integer_exact(csa):
    wl = Workload("fp8", B=1, S=2000, m=4, H=64, D=128, k=128, dist="int", dtype="e4m3fn")
    _check(csa, wl, seed=5)


@pytest.mark.parametrize("key_tile", [64, 128, 256])
def test_fp8_key_tiles_integer_exact(csa, key_tile):
    """Every staged key tile of the fp8 kernel (256 is its default), on
    integer inputs whose key count is no multiple of any tile, every row
    exact."""
    wl = Workload("fp8-tiles", B=2, S=3001, m=4, H=64, D=128, k=300, dist="int",
                  dtype="e4m3fn", T=700)
    _check(csa, wl, seed=11, key_tile=key_tile)


def test_fp8_gauss_all_rows(csa):
    wl = Workload("fp8g", B=1, S=2048, m=4, H=64, D=128, k=128, dtype="e4m3fn")
    _, _, stats = _check(csa, wl, seed=6)
    print(stats)


def test_s16k_all_rows(csa):
    """The S=16,384 workload (k = 512), every one of its 16,384 rows
    against the oracle."""
    wl = WORKLOADS["s16k"]
    _, _, stats = _check(csa, wl)
    print(stats)


def test_max_k_many_rows(csa):
    """k = 16,384 (the largest supported): rows sorted by the 256-thread LDS
    sort in 128 KB of LDS; sampled rows around n_vis = k, exact."""
    wl = Workload("maxk", B=1, S=20000, m=1, H=4, D=32, k=16384, dist="int")
    rng = np.random.default_rng(16384)
    rows = np.unique(np.r_[[0, 1, 100, 16382, 16383, 16384, 16385, 19998, 19999],
                           rng.choice(20000, size=40, replace=False)])
    _check(csa, wl, seed=3, rows=rows)


def test_max_k_few_rows(csa):
    """k = 16,384 with fewer rows than compute units: the 1,024-thread LDS
    sort; every row sees about 19,000 keys; all rows exact."""
    wl = Workload("maxk-few", B=1, S=40, m=1, H=4, D=32, k=16384, dist="int", T=20000,
                  row_offset=19000)
    print(f"\n[case] {wl}", flush=True)
    inp = make_inputs(wl, seed=4, device="cuda")
    out_idx, out_score = _run(csa, inp, wl, row_offset=wl.row_offset)
    view = OracleView(inp, wl, 0)
    rows = np.arange(wl.S, dtype=np.int64)
    o_idx, o_score = view.topk(rows, rows + wl.row_offset, wl.k, wl.m)
    compare_exact(out_idx[0].cpu().numpy(), out_score[0].cpu().numpy(), o_idx, o_score,
                  rows + wl.row_offset)
