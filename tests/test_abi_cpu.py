"""C-ABI checks that need no GPU: exported symbols, planning, validation.

Every entry point validates its arguments before it touches the device,
so invalid calls return their documented status here too.
"""
import ctypes
import os
import re

import pytest

import streaming_top_selection_csa_amd as csa
from streaming_top_selection_csa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa_index.h")


@pytest.fixture(scope="module")
def lib():
    return csa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def opts(**kw):
    kw.setdefault("num_cus", 256)
    return B.make_options(**kw)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert csa.status_string(code)
    assert csa.status_string(12345) == "unknown status"


@pytest.mark.parametrize("S,T", [(65536, 16384), (262144, 65536), (1048576, 262144), (1000, 3)])
def test_workspace_independent_of_S_and_T(lib, S, T):
    ref = csa.plan_query(csa.make_desc(1, 65536, 16384, 64, 128), 4, 2048, opts())
    info = csa.plan_query(csa.make_desc(1, S, T, 64, 128), 4, 2048, opts())
    if (S + 7) // 8 >= 256:  # enough blocks to fill the 256-workgroup grid
        assert info.workspace_bytes == ref.workspace_bytes
    assert info.workspace_bytes <= ref.workspace_bytes
    assert info.n_blocks == (S + info.queries_per_block - 1) // info.queries_per_block


def test_plan_fields(lib):
    info = csa.plan_query(csa.make_desc(2, 1000, 250, 4, 32), 4, 64, opts())
    assert info.queries_per_block == 8 * 64 // 4           # 8 waves x 64 rows / H
    assert info.n_blocks == 2 * ((1000 + 127) // 128)
    assert info.grid == min(info.n_blocks, 256)
    assert info.keys_per_tile == 64
    assert info.chunk_keys == 1024                          # default: 4k within [1024, 8192]
    assert info.log_capacity == 64 + 1024
    big = csa.plan_query(csa.make_desc(1, 4096, 1024, 64, 128), 4, 2048, opts())
    assert big.chunk_keys == 8192 and big.log_capacity == 2048 + 8192
    c = csa.plan_query(csa.make_desc(1, 4096, 1024, 64, 128), 4, 100, opts(chunk_keys=100))
    assert c.chunk_keys == 128                              # rounded up to the tile
    assert csa.workspace_bytes(csa.make_desc(1, 4096, 1024, 64, 128), 4, 2048, opts()) == \
        big.workspace_bytes
    assert big.workspace_bytes == 256 * 8 * 1 * (2048 + 8192) * 8


def bad(lib, desc, m=4, k=8, opt=None):
    info = B.CsaPlanInfo()
    o = opt if opt is not None else opts()
    return lib.csa_plan_query(ctypes.byref(desc) if desc is not None else None, m, k,
                              ctypes.byref(o), ctypes.byref(info))


def test_validation_errors(lib):
    ok = csa.make_desc(1, 100, 25, 64, 128)
    assert bad(lib, ok) == B.CSA_OK
    assert bad(lib, None) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, ok, m=0) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, ok, k=0) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, ok, k=16385) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, csa.make_desc(0, 100, 25, 64, 128)) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, csa.make_desc(1, -1, 25, 64, 128)) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, csa.make_desc(1, 100, -1, 64, 128)) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, csa.make_desc(1, 100, 25, 3, 128)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, csa.make_desc(1, 100, 25, 128, 128)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, csa.make_desc(1, 100, 25, 64, 48)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, csa.make_desc(1, 100, 25, 64, 32, B.CSA_FP8_E4M3FN, 1, 1)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, csa.make_desc(1, 100, 25, 64, 128, 7)) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, csa.make_desc(1, 100, 25, 64, 128, B.CSA_FP8_E4M3FN)) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, csa.make_desc(1, 100, 25, 64, 128, B.CSA_BF16, 16, 0)) == B.CSA_ERR_INVALID_ARG
    d = csa.make_desc(1, 100, 25, 64, 128)
    d.reserved0 = 1
    assert bad(lib, d) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, ok, opt=opts(row_offset=-1)) == B.CSA_ERR_INVALID_ARG
    assert bad(lib, ok, opt=opts(chunk_keys=-5)) == B.CSA_ERR_INVALID_ARG
    o = opts()
    o.num_cus = -1
    assert bad(lib, ok, opt=o) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_plan_query(ctypes.byref(ok), 4, 8, ctypes.byref(opts()), None) == \
        B.CSA_ERR_INVALID_ARG
    assert lib.csa_workspace_bytes(ctypes.byref(csa.make_desc(1, 100, 25, 3, 128)), 4, 8,
                                   ctypes.byref(opts())) == 0


def call_index(lib, q=16, w=16, k_cmp=16, oi=16, os_=16, desc=None, opt=None, m=4, k=8):
    desc = desc or csa.make_desc(1, 100, 25, 64, 128)
    opt = opt or opts()
    return lib.csa_index_ex(q, w, k_cmp, ctypes.byref(desc), m, k, oi, os_,
                            ctypes.byref(opt), None)


def test_index_rejects_before_touching_the_device(lib):
    # dummy (never dereferenced) addresses: every call below must fail validation
    assert call_index(lib, q=None) == B.CSA_ERR_INVALID_ARG
    assert call_index(lib, w=None) == B.CSA_ERR_INVALID_ARG
    assert call_index(lib, k_cmp=None) == B.CSA_ERR_INVALID_ARG
    assert call_index(lib, oi=None) == B.CSA_ERR_INVALID_ARG
    # out_score = NULL is valid (no scores returned): it gets as far as the
    # workspace check, still before any device work
    assert call_index(lib, os_=None, opt=opts(workspace=256, workspace_bytes=1024)) == \
        B.CSA_ERR_WORKSPACE
    assert call_index(lib, q=24) == B.CSA_ERR_INVALID_ARG          # q not 16-byte aligned
    assert call_index(lib, k_cmp=40) == B.CSA_ERR_INVALID_ARG
    assert call_index(lib, w=18) == B.CSA_ERR_INVALID_ARG
    assert call_index(lib, k=0) == B.CSA_ERR_INVALID_ARG
    short = opts(workspace=256, workspace_bytes=1024)
    assert call_index(lib, opt=short) == B.CSA_ERR_WORKSPACE
    misaligned = opts(workspace=272, workspace_bytes=1 << 40)
    assert call_index(lib, opt=misaligned) == B.CSA_ERR_WORKSPACE
    # nothing to do: no rows
    assert call_index(lib, q=None, w=None, oi=None, os_=None,
                      desc=csa.make_desc(1, 0, 25, 64, 128)) == B.CSA_OK


def test_binding_refuses_host_tensors(lib):
    import torch
    q = torch.zeros((1, 8, 64, 128), dtype=torch.bfloat16)
    w = torch.zeros((1, 8, 64), dtype=torch.float32)
    k = torch.zeros((1, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        csa.index(q, w, k, 4, 2)


def test_key_splits_plan(lib):
    """Key ranges appear only when the query blocks leave compute units idle,
    and the workspace then holds B*S*G*k partial entries."""
    # 64 positions at the end of a 262,144-position context, 65,536 keys
    dec = csa.make_desc(1, 64, 65536, 64, 128)
    info = csa.plan_query(dec, 4, 2048, opts(row_offset=4 * 65536 - 64))
    assert info.n_blocks == 8
    assert info.key_splits == 28                       # min(256/8, 65536/(2048 + 256))
    assert info.grid == 8 * 28
    logs = 8 * 28 * 8 * (2048 + 8192) * 8
    assert info.workspace_bytes == logs + 64 * 28 * 2048 * 8
    # early positions see few keys: no range below max(9k/8, 1024) keys
    early = csa.plan_query(dec, 4, 2048, opts(row_offset=0))
    assert early.key_splits == 1 and early.workspace_bytes == 256 * 8 * (2048 + 8192) * 8 // 32
    # enough query blocks: never split
    big = csa.plan_query(csa.make_desc(1, 65536, 16384, 64, 128), 4, 2048, opts())
    assert big.key_splits == 1
    # requested ranges: at most one per 64 visible keys
    assert csa.plan_query(dec, 4, 2048, opts(row_offset=262080, key_splits=5)).key_splits == 5
    assert csa.plan_query(dec, 4, 2048, opts(row_offset=262080, key_splits=1)).key_splits == 1
    few = csa.plan_query(csa.make_desc(1, 8, 100, 64, 128), 4, 16, opts(row_offset=1000,
                                                                        key_splits=50))
    assert few.key_splits == 2                         # 100 keys -> 2 tiles
    # automatic ranges keep the partial lists under 1 GiB, requested ones
    # under 64 GiB: G is lowered
    auto = csa.plan_query(csa.make_desc(1, 64, 65536, 64, 128), 4, 16384, opts(row_offset=262080))
    assert 64 * auto.key_splits * 16384 * 8 <= 1 << 30
    wide = csa.plan_query(csa.make_desc(1, 65536, 65536, 64, 128), 4, 16384,
                          opts(row_offset=262144, key_splits=64))
    assert 65536 * wide.key_splits * 16384 * 8 <= 1 << 36 and wide.key_splits == 8
    # the key-range sweep of the S=65,536 workload: 16 ranges of 1,024 keys
    sweep = csa.plan_query(csa.make_desc(1, 65536, 16384, 64, 128), 4, 2048, opts(key_splits=16))
    assert sweep.key_splits == 16


def test_key_splits_validation(lib):
    ok = csa.make_desc(1, 100, 25, 64, 128)
    assert bad(lib, ok, opt=opts(key_splits=-1)) == B.CSA_ERR_INVALID_ARG
    o = opts()
    o.flags = 3
    assert bad(lib, ok, opt=o) == B.CSA_ERR_INVALID_ARG


def test_bench_visible_pairs_closed_form():
    """bench.py's closed-form count of visible (position, key) pairs against
    the direct sum over positions."""
    import bench
    for S, T, m, off in [(1024, 256, 4, 0), (1000, 250, 4, 0), (777, 300, 3, 0), (90, 40, 1, 0),
                         (64, 65536, 4, 4 * 65536 - 64), (300, 50, 2, 17), (5, 0, 4, 0),
                         (4096, 2000, 4, 100)]:
        direct = sum(min(T, (t + 1) // m) for t in range(off, off + S))
        assert bench.visible_pairs(S, T, m, 1, off) == direct, (S, T, m, off)
    # the headline shape: m*T*(T-1)/2 + T with S = m*T
    assert bench.visible_pairs(262144, 65536, 4) == 4 * 65536 * 65535 // 2 + 65536


def attn_call(lib, desc, scale=0.125, q=16, k=16, v=16, idx=16, out=16, lse=None):
    """csa_sparse_attention with fake (never dereferenced) pointers: every
    case below must be rejected before anything touches the device."""
    vp = ctypes.c_void_p
    return lib.csa_sparse_attention(vp(q) if q else None, vp(k) if k else None,
                                    vp(v) if v else None, vp(idx) if idx else None,
                                    ctypes.byref(desc) if desc is not None else None,
                                    ctypes.c_float(scale), vp(out) if out else None,
                                    vp(lse) if lse else None, None)


def test_sparse_attention_validation(lib):
    E = B.CSA_ERR_INVALID_ARG
    U = B.CSA_ERR_UNSUPPORTED
    ok = csa.make_attn_desc(1, 4, 10, 64, 128, 8)
    assert attn_call(lib, None) == E
    for H, D in [(16, 128), (64, 32), (96, 128), (64, 256), (1, 64)]:
        assert attn_call(lib, csa.make_attn_desc(1, 4, 10, H, D, 8)) == U, (H, D)
    for args in [(0, 4, 10, 64, 128, 8), (1, -1, 10, 64, 128, 8), (1, 4, -1, 64, 128, 8),
                 (1, 4, 10, 64, 128, -1)]:
        assert attn_call(lib, csa.make_attn_desc(*args)) == E, args
    r = csa.make_attn_desc(1, 4, 10, 64, 128, 8)
    r.reserved0 = 1
    assert attn_call(lib, r) == E
    assert attn_call(lib, ok, scale=float("nan")) == E
    assert attn_call(lib, ok, scale=float("inf")) == E
    assert attn_call(lib, ok, q=0) == E
    assert attn_call(lib, ok, out=0) == E
    assert attn_call(lib, ok, idx=0) == E
    assert attn_call(lib, ok, k=0) == E and attn_call(lib, ok, v=0) == E
    assert attn_call(lib, ok, q=24) == E      # not 16-byte aligned
    assert attn_call(lib, ok, out=8) == E
    assert attn_call(lib, ok, idx=18) == E    # not 4-byte aligned
    assert attn_call(lib, ok, lse=2) == E
    # sizes whose byte offsets would overflow
    assert attn_call(lib, csa.make_attn_desc(1 << 20, 1 << 40, 10, 64, 128, 8)) == E
    # nothing to do: no rows (no pointer is needed)
    assert attn_call(lib, csa.make_attn_desc(1, 0, 10, 64, 128, 8), q=0, k=0, v=0, idx=0,
                     out=0) == B.CSA_OK


def attn_plan(desc, **kw):
    kw.setdefault("num_cus", 256)
    return csa.attention_plan(desc, csa.make_attn_options(**kw))


def test_sparse_attention_split_plan(lib):
    dec = csa.make_attn_desc(1, 64, 65536, 64, 128, 2048)
    # 64 rows on 256 CUs: ranges of at least 512 entries toward 4 workgroups per CU
    assert attn_plan(dec, entry_splits=0) == (4, 64 * 4 * 64 * 130 * 4)
    assert attn_plan(dec, entry_splits=1) == (1, 0)
    assert attn_plan(dec, entry_splits=5)[0] == 5            # 64 tiles -> ranges of 13 tiles
    assert attn_plan(dec, entry_splits=100)[0] == 64         # at most one range per tile
    assert attn_plan(dec, entry_splits=0, num_cus=8)[0] == 1  # 64 rows already fill 8 CUs
    big = csa.make_attn_desc(1, 262144, 65536, 64, 128, 2048)
    assert attn_plan(big, entry_splits=0) == (1, 0)
    assert attn_plan(csa.make_attn_desc(1, 4, 100, 64, 128, 20), entry_splits=0)[0] == 1
    assert attn_plan(csa.make_attn_desc(1, 4, 0, 64, 128, 2048), entry_splits=0)[0] == 1
    # the workspace query writes the split count
    g = ctypes.c_int32(-7)
    n = lib.csa_sparse_attention_workspace_bytes(ctypes.byref(dec), ctypes.byref(
        csa.make_attn_options(3, 256)), ctypes.byref(g))
    assert g.value == 3 and n == 64 * 3 * 64 * 130 * 4


def test_sparse_attention_ex_validation(lib):
    E = B.CSA_ERR_INVALID_ARG
    dec = csa.make_attn_desc(1, 64, 65536, 64, 128, 2048)
    vp = ctypes.c_void_p

    def call(opt):
        return lib.csa_sparse_attention_ex(vp(16), vp(16), vp(16), vp(16), ctypes.byref(dec),
                                           ctypes.c_float(0.1), vp(16), None, ctypes.byref(opt),
                                           None)
    assert call(csa.make_attn_options(-1, 256)) == E
    assert call(csa.make_attn_options(1, -3)) == E
    o = csa.make_attn_options(4, 256)
    o.reserved = 1
    assert call(o) == E
    # a caller workspace smaller than the plan, or misaligned
    need = attn_plan(dec, entry_splits=4)[1]
    assert call(csa.make_attn_options(4, 256, 256, need - 1)) == B.CSA_ERR_WORKSPACE
    assert call(csa.make_attn_options(4, 256, 256 + 64, need)) == B.CSA_ERR_WORKSPACE
    assert lib.csa_sparse_attention_workspace_bytes(None, None, None) == 0


def test_header_is_plain_c(tmp_path):
    """include/csa_index.h compiles as C99 and C++17 on its own (with only
    the HIP runtime API header) and every declared entry point is callable
    with the documented argument types."""
    import shutil
    import subprocess
    rocm_inc = "/opt/rocm/include"
    if not os.path.isdir(rocm_inc) or shutil.which("gcc") is None:
        pytest.skip("no ROCm headers or gcc")
    src = tmp_path / "use.c"
    src.write_text('''#include "csa_index.h"
int use(void) {
    csa_desc d = {1, 16, 4, 64, 128, CSA_BF16, 0, 0, 0};
    csa_options o = {0};
    csa_plan_info info;
    csa_attn_desc ad = {1, 16, 4, 64, 128, 8, 0};
    csa_attn_options ao = {0};
    int32_t g = 0;
    size_t n = csa_workspace_bytes(&d, 4, 8, &o) + csa_sparse_attention_workspace_bytes(&ad, &ao, &g);
    int rc = csa_plan_query(&d, 4, 8, &o, &info);
    rc |= csa_index(0, 0, 0, &d, 4, 8, 0, 0, 0) | csa_index_ex(0, 0, 0, &d, 4, 8, 0, 0, &o, 0);
    rc |= csa_sparse_attention(0, 0, 0, 0, &ad, 0.1f, 0, 0, 0);
    rc |= csa_sparse_attention_ex(0, 0, 0, 0, &ad, 0.1f, 0, 0, &ao, 0);
    return rc + (int)n + (csa_status_string(rc) != 0);
}
''')
    for compiler, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        cmd = [compiler, std, "-x", "c" if compiler == "gcc" else "c++", "-fsyntax-only",
               "-Wall", "-Wextra", "-Werror", "-Wno-missing-field-initializers",
               "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
               "-I", rocm_inc, str(src)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with a message
    before anything touches a device."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_host_code_fuzz_under_sanitizers(tmp_path):
    """The planning and validation code of the C ABI, built for the host
    with AddressSanitizer and UBSan (no device code: the HIP runtime and
    the kernel launchers are stubbed), survives 200,000 random, extreme and
    hostile argument sets with consistent plans."""
    import shutil
    import subprocess
    rocm_inc = "/opt/rocm/include"
    if not os.path.isdir(rocm_inc) or shutil.which("g++") is None:
        pytest.skip("no ROCm headers or g++")
    csrc = os.path.join(ROOT, "streaming_top_selection_csa_amd", "csrc")
    exe = tmp_path / "fuzz_abi_host"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", rocm_inc,
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "fuzz_abi_host.cpp"), os.path.join(csrc, "csa_plan.cpp"),
           os.path.join(csrc, "csa_abi.cpp"), os.path.join(csrc, "csa_grouped.cpp"), "-o",
           str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe), "200000"], capture_output=True, text=True, timeout=300,
                         env=env)
    assert res.returncode == 0, (res.stdout + res.stderr)[-3000:]
    assert "fuzz ok" in res.stdout


def test_no_score_workspace_sizes(lib):
    """CSA_FLAG_NO_SCORE sizes the workspace for out_score = NULL: nothing
    extra when the scoring kernel sorts the rows (next_pow2(k) <= 2048, no
    key ranges) or the merge kernel does (key ranges, fewer rows than
    compute units), B*S*k*4 more bytes when a separate pass sorts them."""
    d = csa.make_desc(1, 100000, 25000, 64, 128)
    ns = opts(flags=csa.CSA_FLAG_NO_SCORE)
    assert csa.workspace_bytes(d, 4, 2048, ns) == csa.workspace_bytes(d, 4, 2048, opts())
    assert (csa.workspace_bytes(d, 4, 4096, ns) - csa.workspace_bytes(d, 4, 4096, opts())
            == 100000 * 4096 * 4)
    few = csa.make_desc(1, 64, 65536, 64, 128)
    o = opts(row_offset=262080, key_splits=8)
    o_ns = opts(row_offset=262080, key_splits=8, flags=csa.CSA_FLAG_NO_SCORE)
    assert csa.workspace_bytes(few, 4, 2048, o_ns) == csa.workspace_bytes(few, 4, 2048, o)
    many = csa.make_desc(1, 4096, 16384, 64, 128)
    o = opts(key_splits=4)
    o_ns = opts(key_splits=4, flags=csa.CSA_FLAG_NO_SCORE)
    assert csa.workspace_bytes(many, 4, 2048, o_ns) - csa.workspace_bytes(many, 4, 2048, o) == \
        4096 * 2048 * 4
    # other flag bits are invalid
    assert csa.workspace_bytes(d, 4, 2048, opts(flags=2)) == 0


def test_key_count_bound(lib):
    """T is limited to 2^30 compressed keys (the kernels' key arithmetic is
    32-bit)."""
    ok = csa.make_desc(1, 16, 1 << 30, 64, 128)
    assert csa.plan_query(ok, 4, 16, opts()).grid >= 1
    assert bad(lib, csa.make_desc(1, 16, (1 << 30) + 1, 64, 128)) == B.CSA_ERR_INVALID_ARG


def test_static_entry_point_validation(lib):
    """csa_index_static rejects a caller workspace and a call whose
    workspace cannot fit its fixed scratch, before touching the device."""
    d = csa.make_desc(1, 100, 25, 64, 128)
    o = opts(workspace=256, workspace_bytes=1 << 20)
    assert lib.csa_index_static(16, 16, 16, ctypes.byref(d), 4, 8, 16, 16, ctypes.byref(o),
                                None) == B.CSA_ERR_INVALID_ARG
    # k = 16,384 rows: candidate logs of 256 * 8 * (16,384 + 64) * 8 bytes even
    # at the smallest partition, more than the 128 MiB scratch
    big = csa.make_desc(1, 1 << 20, 1 << 18, 64, 128)
    assert lib.csa_index_static(16, 16, 16, ctypes.byref(big), 4, 16384, 16, 16,
                                ctypes.byref(opts()), None) == B.CSA_ERR_WORKSPACE
    assert lib.csa_index_static(16, 16, 16, ctypes.byref(d), 0, 8, 16, 16,
                                ctypes.byref(opts()), None) == B.CSA_ERR_INVALID_ARG


def test_key_tile_option(lib):
    """Staged key tiles other than 64 exist for H = 64, D = 128: rows sorted
    by the scoring kernel (bf16: 32 to 256; fp8: 128 and 256), and the
    unsorted kernel (bf16: 128); elsewhere they are unsupported."""
    d = csa.make_desc(1, 65536, 16384, 64, 128)
    for kt in (32, 64, 128, 192, 256):
        assert csa.plan_query(d, 4, 2048, opts(key_tile=kt)).keys_per_tile == kt
    assert csa.plan_query(d, 4, 2048, opts()).keys_per_tile == 128   # default for this shape
    assert csa.plan_query(d, 4, 4096, opts()).keys_per_tile == 128   # rows sorted separately
    assert csa.plan_query(d, 4, 4096, opts(key_tile=64)).keys_per_tile == 64
    assert csa.plan_query(csa.make_desc(1, 100, 25, 32, 128), 4, 8, opts()).keys_per_tile == 64
    f8 = csa.make_desc(1, 65536, 16384, 64, 128, B.CSA_FP8_E4M3FN, 16, 16)
    assert csa.plan_query(f8, 4, 2048, opts()).keys_per_tile == 256   # fp8 default
    for kt in (64, 128, 256):
        assert csa.plan_query(f8, 4, 2048, opts(key_tile=kt)).keys_per_tile == kt
    assert bad(lib, f8, k=2048, opt=opts(key_tile=192)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, f8, k=2048, opt=opts(key_tile=32)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, d, k=2048, opt=opts(key_tile=96)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, d, k=4096, opt=opts(key_tile=192)) == B.CSA_ERR_UNSUPPORTED  # separate sort
    assert bad(lib, d, k=2048, opt=opts(key_tile=256, key_splits=4)) == B.CSA_ERR_UNSUPPORTED
    assert csa.plan_query(d, 4, 2048, opts(key_splits=4)).keys_per_tile == 128
    assert bad(lib, f8, k=4096, opt=opts(key_tile=128)) == B.CSA_ERR_UNSUPPORTED
    assert bad(lib, csa.make_desc(1, 100, 25, 32, 128), opt=opts(key_tile=128)) == \
        B.CSA_ERR_UNSUPPORTED
    assert bad(lib, d, opt=opts(key_tile=-64)) == B.CSA_ERR_INVALID_ARG
    o = opts()
    o.reserved2 = 1
    assert bad(lib, d, opt=o) == B.CSA_ERR_INVALID_ARG


def _unit_coverage(desc, m, k, opt):
    """Walks the scoring kernel's work decomposition for a plan: the
    persistent grid's dealing of units (XCD-grouped, snake order) and each
    unit's (query block, key range); checks that every unit is dealt once
    and every causally visible (b, t, s) pair is scored exactly once."""
    import numpy as np
    info = csa.plan_query(desc, m, k, opt)
    B, S, T, off = desc.B, desc.S, desc.T, opt.row_offset
    QB, G, grid = info.queries_per_block, info.key_splits, info.grid
    R = info.keys_per_range if G > 1 else 1 << 30
    bpb = -(-S // QB)
    n_units = bpb * B * G
    assert info.n_blocks == bpb * B
    dealt = np.zeros(n_units, np.int64)
    per_xcd = grid >> 3
    for g in range(grid):
        xcd, in_xcd = g & 7, g >> 3
        rnd = 0
        while True:
            if grid & 7:
                j = rnd * grid + ((grid - 1 - g) if rnd & 1 else g)
            else:
                j = (rnd * 8 + ((7 - xcd) if rnd & 1 else xcd)) * per_xcd + in_xcd
            if j >= n_units:
                break
            dealt[j] += 1
            rnd += 1
    assert (dealt == 1).all()
    nvis = lambda t: np.minimum(T, (t + 1) // m)
    covered = np.zeros((B, S), np.int64)
    ends = np.zeros((B, S), np.int64)       # next key each position expects
    for j in range(n_units):
        jq, js = j // G, j % G
        b, blk = jq % B, bpb - 1 - jq // B
        p0 = blk * QB
        pos = np.arange(p0, min(p0 + QB, S))
        klo = js * R
        hi = min(int(nvis(off + pos[-1])), klo + R)
        lo_t = np.full(pos.shape, klo)
        hi_t = np.minimum(nvis(off + pos), hi)
        n = np.maximum(hi_t - lo_t, 0)
        # ranges of one position come in ascending, contiguous order
        assert ((n == 0) | (lo_t == ends[b, pos])).all()
        ends[b, pos] = np.where(n > 0, hi_t, ends[b, pos])
        covered[b, pos] += n
    want = nvis(off + np.arange(S))
    assert (covered == want[None, :]).all()


@pytest.mark.parametrize("B,S,T,m,k,off,splits", [
    (1, 262144, 65536, 4, 2048, 0, 0),          # the headline shape, no ranges
    (1, 64, 65536, 4, 2048, 262080, 0),         # decode: automatic ranges
    (32, 4, 16384, 4, 2048, 65532, 0),          # 32 sequences of 4 positions
    (2, 3001, 500, 3, 100, 7, 0),               # ragged blocks, T < S/m
    (1, 64, 65536, 4, 2048, 262080, 7),         # requested ranges
    (1, 5000, 1250, 4, 64, 0, 3),
    (3, 777, 100, 1, 16, 0, 0),                 # m = 1
])
def test_planner_covers_every_visible_pair_once(lib, B, S, T, m, k, off, splits):
    _unit_coverage(csa.make_desc(B, S, T, 64, 128), m, k,
                   opts(row_offset=off, key_splits=splits))
