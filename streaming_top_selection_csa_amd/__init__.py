"""MI355X-native CSA lightning-indexer top-k (streaming partition-merge) and
the sparse attention over the selected keys.

The compute lives in libcsa_index.so (hand-written gfx950 HIP kernels behind
the C ABI in include/csa_index.h); this package is its Python binding.
Importing it loads nothing; the library is loaded on first use and calls
fail loudly if it is missing.
"""
from .binding import (CSA_BF16, CSA_FLAG_NO_SCORE, CSA_FP8_E4M3FN, STATIC_SCRATCH_BYTES,
                      CsaError, HipEvents, attention_plan, attention_workspace_for,
                      grouped_workspace_bytes, grouped_workspace_for, index, index_grouped,
                      load_library, make_attn_desc, make_attn_options, make_desc,
                      make_group_options, make_options, plan_query, sparse_attention,
                      status_string, workspace_bytes, workspace_for)

__all__ = ["index", "index_grouped", "grouped_workspace_for", "grouped_workspace_bytes",
           "make_group_options", "sparse_attention", "make_attn_desc", "make_attn_options", "attention_plan",
           "attention_workspace_for", "plan_query", "workspace_bytes", "workspace_for", "load_library",
           "status_string", "make_desc", "make_options", "CsaError", "HipEvents",
           "CSA_BF16", "CSA_FP8_E4M3FN", "CSA_FLAG_NO_SCORE", "STATIC_SCRATCH_BYTES"]
