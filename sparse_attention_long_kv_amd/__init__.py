"""MI355X (gfx950) indexer-selected token-sparse decode: a C-ABI HIP library
(libsparse_attn.so, declared in include/sparse_attn.h) and its thin ctypes
binding.  See ``_lib`` for the functions; build with
``python -m sparse_attention_long_kv_amd.build_lib``.
"""

from ._lib import (  # noqa: F401
    SaShape, SparseAttnError, make_shape, load, exported_symbols, alloc_workspace,
    sparse_attn_append_kv, sparse_attn_project_keys, sparse_attn_index_score,
    sparse_attn_topm, sparse_attn_index_topm, sparse_attn_index_topm_stage,
    SA_STAGE_BOUND, SA_STAGE_CANDIDATES, SA_STAGE_MERGE, sparse_attn_decode,
    sparse_attn_decode_step, sparse_attn_decode_step_stage, sparse_attn_decode_step_noalloc,
    SA_STEP_APPEND_BOUND, SA_STEP_CANDIDATES, SA_STEP_MERGE, SA_STEP_ATTEND,
    SA_STEP_SELECT_ATTEND,
    sparse_attn_linear_gate, sparse_attn_dense_decode, sparse_attn_dense_workspace_size,
    sparse_attn_gather_kv, sparse_attn_stream_read, sparse_attn_row_read, sparse_attn_selection_fallbacks,
    sparse_attn_selection_plan, SA_PLAN_CHUNK_EXACT, SA_PLAN_FILTER, SA_PLAN_UNIT,
    SA_PLAN_SCORES,
    sparse_attn_workspace_size, sparse_attn_status_string, LIB_PATH,
    SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP,
    SA_ERR_TOO_LARGE, SA_NOALLOC_SCRATCH_BYTES,
)
