"""ctypes binding of libcsa_index.so (argument marshalling only).

Every step of the indexer runs in the HIP library; this module only turns
torch device tensors into the pointers and sizes of the C ABI declared in
include/csa_index.h, allocates outputs with torch when the caller gives
none, and raises on a non-zero status.  There is no fallback: without the
built library or without a GPU tensor, calls fail.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa_index.so")

CSA_OK = 0
CSA_ERR_INVALID_ARG = -1
CSA_ERR_UNSUPPORTED = -2
CSA_ERR_WORKSPACE = -3
CSA_ERR_HIP = -4

CSA_BF16 = 0
CSA_FP8_E4M3FN = 1

CSA_FLAG_NO_SCORE = 1

EXPORTS = ("csa_index", "csa_index_ex", "csa_index_static", "csa_index_grouped",
           "csa_grouped_workspace_bytes", "csa_workspace_bytes", "csa_plan_query",
           "csa_status_string", "csa_sparse_attention", "csa_sparse_attention_ex",
           "csa_sparse_attention_workspace_bytes")


class CsaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S", ctypes.c_int64), ("T", ctypes.c_int64),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("q_scale", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p)]


class CsaOptions(ctypes.Structure):
    _fields_ = [("chunk_keys", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("row_offset", ctypes.c_int64), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("timing", ctypes.c_void_p * 2),
                ("key_splits", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("key_tile", ctypes.c_int32), ("reserved2", ctypes.c_int32)]


class CsaPlanInfo(ctypes.Structure):
    _fields_ = [("queries_per_block", ctypes.c_int32), ("keys_per_tile", ctypes.c_int32),
                ("chunk_keys", ctypes.c_int32), ("log_capacity", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("key_splits", ctypes.c_int32),
                ("n_blocks", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("keys_per_range", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class CsaGroupOptions(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("candidates", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


class CsaAttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S", ctypes.c_int64), ("T", ctypes.c_int64),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("n_sel", ctypes.c_int32),
                ("reserved0", ctypes.c_int32)]


class CsaAttnOptions(ctypes.Structure):
    _fields_ = [("entry_splits", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("reserved", ctypes.c_int64)]


class CsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load_library():
    """Load libcsa_index.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m streaming_top_selection_csa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.csa_index.argtypes = [vp, vp, vp, ctypes.POINTER(CsaDesc), i32, i32, vp, vp, vp]
    lib.csa_index.restype = ctypes.c_int
    lib.csa_index_ex.argtypes = [vp, vp, vp, ctypes.POINTER(CsaDesc), i32, i32, vp, vp,
                                 ctypes.POINTER(CsaOptions), vp]
    lib.csa_index_ex.restype = ctypes.c_int
    lib.csa_index_static.argtypes = lib.csa_index_ex.argtypes
    lib.csa_index_static.restype = ctypes.c_int
    lib.csa_index_grouped.argtypes = [vp, vp, vp, ctypes.POINTER(CsaDesc), i32, i32,
                                      ctypes.POINTER(CsaGroupOptions), vp, vp,
                                      ctypes.POINTER(CsaOptions), vp]
    lib.csa_index_grouped.restype = ctypes.c_int
    lib.csa_grouped_workspace_bytes.argtypes = [ctypes.POINTER(CsaDesc), i32, i32,
                                                ctypes.POINTER(CsaGroupOptions),
                                                ctypes.POINTER(CsaOptions)]
    lib.csa_grouped_workspace_bytes.restype = ctypes.c_size_t
    lib.csa_workspace_bytes.argtypes = [ctypes.POINTER(CsaDesc), i32, i32,
                                        ctypes.POINTER(CsaOptions)]
    lib.csa_workspace_bytes.restype = ctypes.c_size_t
    lib.csa_plan_query.argtypes = [ctypes.POINTER(CsaDesc), i32, i32, ctypes.POINTER(CsaOptions),
                                   ctypes.POINTER(CsaPlanInfo)]
    lib.csa_plan_query.restype = ctypes.c_int
    lib.csa_sparse_attention.argtypes = [vp, vp, vp, vp, ctypes.POINTER(CsaAttnDesc),
                                         ctypes.c_float, vp, vp, vp]
    lib.csa_sparse_attention.restype = ctypes.c_int
    lib.csa_sparse_attention_ex.argtypes = [vp, vp, vp, vp, ctypes.POINTER(CsaAttnDesc),
                                            ctypes.c_float, vp, vp,
                                            ctypes.POINTER(CsaAttnOptions), vp]
    lib.csa_sparse_attention_ex.restype = ctypes.c_int
    lib.csa_sparse_attention_workspace_bytes.argtypes = [
        ctypes.POINTER(CsaAttnDesc), ctypes.POINTER(CsaAttnOptions), ctypes.POINTER(ctypes.c_int32)]
    lib.csa_sparse_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.csa_status_string.argtypes = [ctypes.c_int]
    lib.csa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().csa_status_string(int(status)).decode()


def make_desc(B, S, T, H, D, dtype=CSA_BF16, q_scale_ptr=0, k_scale_ptr=0) -> CsaDesc:
    return CsaDesc(int(B), int(S), int(T), int(H), int(D), int(dtype), 0,
                   q_scale_ptr or None, k_scale_ptr or None)


def make_options(chunk_keys=0, row_offset=0, num_cus=0, workspace=None, workspace_bytes=0,
                 timing=(None, None), key_splits=0, flags=0, key_tile=0) -> CsaOptions:
    opt = CsaOptions()
    opt.key_tile = int(key_tile)
    opt.key_splits = int(key_splits)
    opt.flags = int(flags)
    opt.chunk_keys = int(chunk_keys)
    opt.num_cus = int(num_cus)
    opt.row_offset = int(row_offset)
    opt.workspace = workspace or None
    opt.workspace_bytes = int(workspace_bytes)
    opt.timing[0] = timing[0]
    opt.timing[1] = timing[1]
    return opt


def plan_query(desc: CsaDesc, m: int, k: int, opt: Optional[CsaOptions] = None) -> CsaPlanInfo:
    info = CsaPlanInfo()
    rc = load_library().csa_plan_query(ctypes.byref(desc), int(m), int(k),
                                       ctypes.byref(opt) if opt is not None else None,
                                       ctypes.byref(info))
    if rc != CSA_OK:
        raise CsaError(rc, "csa_plan_query")
    return info


STATIC_SCRATCH_BYTES = 128 << 20   # CSA_STATIC_SCRATCH_BYTES


def workspace_bytes(desc: CsaDesc, m: int, k: int, opt: Optional[CsaOptions] = None) -> int:
    return int(load_library().csa_workspace_bytes(
        ctypes.byref(desc), int(m), int(k), ctypes.byref(opt) if opt is not None else None))


def _dtype_code(q: torch.Tensor) -> int:
    if q.dtype == torch.bfloat16:
        return CSA_BF16
    if q.dtype == torch.float8_e4m3fn:
        return CSA_FP8_E4M3FN
    raise TypeError(f"q/k_cmp must be bfloat16 or float8_e4m3fn, got {q.dtype}")


def _check(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def index(q: torch.Tensor, w: torch.Tensor, k_cmp: torch.Tensor, m: int, k: int, *,
          q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
          out_idx: Optional[torch.Tensor] = None, out_score: Optional[torch.Tensor] = None,
          chunk_keys: int = 0, row_offset: int = 0, key_splits: int = 0,
          workspace: Optional[torch.Tensor] = None, timing=None,
          stream: Optional[torch.cuda.Stream] = None, want_score: bool = True,
          static_scratch: bool = False, key_tile: int = 0):
    """Top-k compressed keys per query position (csa_index_ex, or with
    static_scratch=True csa_index_static: no allocation, the library's fixed
    device scratch instead of a workspace; `workspace` must then be None).

    q [B,S,H,D] bf16 | e4m3fn, w [B,S,H] fp32, k_cmp [B,T,D] same dtype as
    q; for fp8 also q_scale [B,S,H] and k_scale [B,T] fp32.  Returns
    (out_idx int32 [B,S,k], out_score fp32 [B,S,k]); with want_score=False
    no score output is passed (out_score = NULL) and the second item is
    None.  `timing` is an optional pair of raw hipEvent_t handles recorded
    around the scoring kernel.  Asynchronous on `stream` (default: torch's
    current stream).
    """
    lib = load_library()
    dt = _dtype_code(q)
    _check(q, "q")
    _check(k_cmp, "k_cmp", q.dtype)
    _check(w, "w", torch.float32)
    if q.dim() != 4 or w.dim() != 3 or k_cmp.dim() != 3:
        raise ValueError("expected q [B,S,H,D], w [B,S,H], k_cmp [B,T,D]")
    B, S, H, D = q.shape
    T = k_cmp.shape[1]
    if tuple(w.shape) != (B, S, H) or k_cmp.shape[0] != B or k_cmp.shape[2] != D:
        raise ValueError("inconsistent shapes of q, w, k_cmp")
    qs_ptr = ks_ptr = 0
    if dt == CSA_FP8_E4M3FN:
        if q_scale is None or k_scale is None:
            raise ValueError("fp8 inputs need q_scale and k_scale")
        _check(q_scale, "q_scale", torch.float32)
        _check(k_scale, "k_scale", torch.float32)
        if tuple(q_scale.shape) != (B, S, H) or tuple(k_scale.shape) != (B, T):
            raise ValueError("q_scale must be [B,S,H] and k_scale [B,T]")
        qs_ptr, ks_ptr = q_scale.data_ptr(), k_scale.data_ptr()
    elif q_scale is not None or k_scale is not None:
        raise ValueError("scales are only used with fp8 inputs")
    if out_idx is None:
        out_idx = torch.empty((B, S, k), dtype=torch.int32, device=q.device)
    if not want_score:
        if out_score is not None:
            raise ValueError("out_score given with want_score=False")
    elif out_score is None:
        out_score = torch.empty((B, S, k), dtype=torch.float32, device=q.device)
    _check(out_idx, "out_idx", torch.int32)
    if tuple(out_idx.shape) != (B, S, k):
        raise ValueError("outputs must be [B,S,k]")
    if out_score is not None:
        _check(out_score, "out_score", torch.float32)
        if tuple(out_score.shape) != (B, S, k):
            raise ValueError("outputs must be [B,S,k]")
    desc = make_desc(B, S, T, H, D, dt, qs_ptr, ks_ptr)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _check(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    opt = make_options(chunk_keys, row_offset, 0, ws_ptr, ws_bytes,
                       timing if timing is not None else (None, None), key_splits,
                       key_tile=key_tile)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    fn = lib.csa_index_static if static_scratch else lib.csa_index_ex
    rc = fn(q.data_ptr(), w.data_ptr(), k_cmp.data_ptr(), ctypes.byref(desc),
            int(m), int(k), out_idx.data_ptr(),
            out_score.data_ptr() if out_score is not None else None,
            ctypes.byref(opt), ctypes.c_void_p(stream.cuda_stream))
    if rc != CSA_OK:
        raise CsaError(rc, "csa_index_static" if static_scratch else "csa_index_ex")
    return out_idx, out_score


def make_group_options(group: int, candidates: int = 0) -> CsaGroupOptions:
    g = CsaGroupOptions()
    g.group = int(group)
    g.candidates = int(candidates)
    return g


def grouped_workspace_bytes(desc: CsaDesc, m: int, k: int, gopt: CsaGroupOptions,
                            opt: Optional[CsaOptions] = None) -> int:
    return int(load_library().csa_grouped_workspace_bytes(
        ctypes.byref(desc), int(m), int(k), ctypes.byref(gopt),
        ctypes.byref(opt) if opt is not None else None))


def index_grouped(q: torch.Tensor, w: torch.Tensor, k_cmp: torch.Tensor, m: int, k: int,
                  group: int, candidates: int = 0, *, out_idx: Optional[torch.Tensor] = None,
                  out_score: Optional[torch.Tensor] = None, want_score: bool = True,
                  row_offset: int = 0, chunk_keys: int = 0,
                  workspace: Optional[torch.Tensor] = None, timing=None,
                  stream: Optional[torch.cuda.Stream] = None):
    """The grouped (approximate) indexer (csa_index_grouped): groups of
    `group` consecutive positions share one scan by their pooled query,
    which keeps `candidates` keys (0 = min(2k, 8192)); each member re-ranks
    them and its own extra keys exactly.  bf16, H = 64, D = 128.  Returns
    (out_idx, out_score or None)."""
    lib = load_library()
    for t, name in ((q, "q"), (k_cmp, "k_cmp")):
        _check(t, name, torch.bfloat16)
    _check(w, "w", torch.float32)
    B, S, H, D = q.shape
    T = k_cmp.shape[1]
    if tuple(w.shape) != (B, S, H) or tuple(k_cmp.shape) != (B, T, D):
        raise ValueError("inconsistent shapes of q, w, k_cmp")
    if out_idx is None:
        out_idx = torch.empty((B, S, k), dtype=torch.int32, device=q.device)
    if want_score and out_score is None:
        out_score = torch.empty((B, S, k), dtype=torch.float32, device=q.device)
    if not want_score and out_score is not None:
        raise ValueError("out_score given with want_score=False")
    _check(out_idx, "out_idx", torch.int32)
    if out_score is not None:
        _check(out_score, "out_score", torch.float32)
    desc = make_desc(B, S, T, H, D)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _check(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    opt = make_options(chunk_keys, row_offset, 0, ws_ptr, ws_bytes,
                       timing if timing is not None else (None, None))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    g = make_group_options(group, candidates)
    rc = lib.csa_index_grouped(q.data_ptr(), w.data_ptr(), k_cmp.data_ptr(), ctypes.byref(desc),
                               int(m), int(k), ctypes.byref(g), out_idx.data_ptr(),
                               out_score.data_ptr() if out_score is not None else None,
                               ctypes.byref(opt), ctypes.c_void_p(stream.cuda_stream))
    if rc != CSA_OK:
        raise CsaError(rc, "csa_index_grouped")
    return out_idx, out_score


def grouped_workspace_for(q: torch.Tensor, k_cmp: torch.Tensor, m: int, k: int, group: int,
                          candidates: int = 0, row_offset: int = 0, chunk_keys: int = 0,
                          want_score: bool = True) -> torch.Tensor:
    """A torch-allocated workspace for `index_grouped` on these inputs."""
    B, S, H, D = q.shape
    n = grouped_workspace_bytes(make_desc(B, S, k_cmp.shape[1], H, D), m, k,
                                make_group_options(group, candidates),
                                make_options(chunk_keys, row_offset,
                                             flags=0 if want_score else CSA_FLAG_NO_SCORE))
    if n == 0:
        raise CsaError(CSA_ERR_INVALID_ARG, "csa_grouped_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def make_attn_desc(B, S, T, H, D, n_sel) -> CsaAttnDesc:
    return CsaAttnDesc(int(B), int(S), int(T), int(H), int(D), int(n_sel), 0)


def make_attn_options(entry_splits=1, num_cus=0, workspace=None, workspace_bytes=0):
    return CsaAttnOptions(int(entry_splits), int(num_cus), workspace, int(workspace_bytes), 0)


def attention_plan(desc: CsaAttnDesc, opt: Optional[CsaAttnOptions] = None):
    """(entry_splits, workspace bytes) csa_sparse_attention_ex would use."""
    g = ctypes.c_int32(0)
    n = load_library().csa_sparse_attention_workspace_bytes(
        ctypes.byref(desc), ctypes.byref(opt) if opt is not None else None, ctypes.byref(g))
    return int(g.value), int(n)


def attention_workspace_for(q: torch.Tensor, k: torch.Tensor, n_sel: int,
                            entry_splits: int = 0) -> torch.Tensor:
    """A torch-allocated workspace big enough for `sparse_attention` with
    this split setting (empty when the rows are not split)."""
    B, S, H, D = q.shape
    _, n = attention_plan(make_attn_desc(B, S, k.shape[1], H, D, n_sel),
                          make_attn_options(entry_splits))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                     scale: Optional[float] = None, *, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                     entry_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None):
    """Softmax attention of every query row over its selected compressed
    entries (csa_sparse_attention_ex).

    q [B,S,H,D] bf16, k and v [B,T,D] bf16, idx [B,S,n_sel] int32 (entries
    outside [0, T) are padding; csa_index's out_idx fits).  `scale`
    multiplies q.k (default 1/sqrt(D)).  `entry_splits`: 1 = one workgroup
    per row (no workspace), 0 = automatic ranges for short query blocks,
    n = n ranges per row; `workspace` holds their partial results (else the
    library allocates it stream-ordered).  Returns (out bf16 [B,S,H,D],
    lse fp32 [B,S,H] or None).  Asynchronous on `stream`.
    """
    lib = load_library()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name, torch.bfloat16)
    _check(idx, "idx", torch.int32)
    if q.dim() != 4 or k.dim() != 3 or v.dim() != 3 or idx.dim() != 3:
        raise ValueError("expected q [B,S,H,D], k and v [B,T,D], idx [B,S,n_sel]")
    B, S, H, D = q.shape
    T = k.shape[1]
    if tuple(k.shape) != (B, T, D) or tuple(v.shape) != (B, T, D) or tuple(idx.shape[:2]) != (B, S):
        raise ValueError("inconsistent shapes of q, k, v, idx")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q.device)
    _check(out, "out", torch.bfloat16)
    if tuple(out.shape) != (B, S, H, D):
        raise ValueError("out must be [B,S,H,D]")
    if lse is None and want_lse:
        lse = torch.empty((B, S, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, S, H):
            raise ValueError("lse must be [B,S,H]")
    desc = make_attn_desc(B, S, T, H, D, idx.shape[2])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _check(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    opt = make_attn_options(entry_splits, 0, ws_ptr, ws_bytes)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    rc = lib.csa_sparse_attention_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                     ctypes.byref(desc), float(scale), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     ctypes.byref(opt), ctypes.c_void_p(stream.cuda_stream))
    if rc != CSA_OK:
        raise CsaError(rc, "csa_sparse_attention_ex")
    return out, lse


def workspace_for(q: torch.Tensor, k_cmp: torch.Tensor, m: int, k: int, chunk_keys: int = 0,
                  row_offset: int = 0, key_splits: int = 0,
                  want_score: bool = True) -> torch.Tensor:
    """A torch-allocated workspace big enough for `index` on these inputs
    (with want_score=False: for calls without a score output)."""
    B, S, H, D = q.shape
    desc = make_desc(B, S, k_cmp.shape[1], H, D, _dtype_code(q),
                     1 if q.dtype == torch.float8_e4m3fn else 0,
                     1 if q.dtype == torch.float8_e4m3fn else 0)
    n = workspace_bytes(desc, m, k, make_options(chunk_keys, row_offset, key_splits=key_splits,
                                                 flags=0 if want_score else CSA_FLAG_NO_SCORE))
    if n == 0:
        raise CsaError(CSA_ERR_INVALID_ARG, "csa_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


class HipEvents:
    """Raw hipEvent_t pairs from the HIP runtime torch already loaded, for
    timing a kernel on the stream it runs on."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(a)) or self._hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a.value, b.value))

    def record(self, event, stream: torch.cuda.Stream):
        """Record raw event `event` on `stream` (hipEventRecord)."""
        if self._hip.hipEventRecord(ctypes.c_void_p(event), ctypes.c_void_p(stream.cuda_stream)):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int) -> float:
        ms = ctypes.c_float()
        a, b = self.pairs[i]
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)):
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for a, b in self.pairs:
            self._hip.hipEventDestroy(ctypes.c_void_p(a))
            self._hip.hipEventDestroy(ctypes.c_void_p(b))
        self.pairs = []
