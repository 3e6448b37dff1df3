"""Exact attention on MI355X (gfx950): RoPE, causal grouped-query prefill, paged-KV decode, MLA absorbed decode,
chunked prefill from a paged cache with RoPE-on-append, and DeepSeek Sparse Attention decode (lightning indexer,
top-k, sparse MLA), as hand-written HIP kernels behind a C ABI (include/attn.h). This package holds the kernels
(csrc/), the build step (build.py) and a thin ctypes binding with the same entry-point names (binding.py).
"""
from .binding import (  # noqa: F401
    AttnError,
    LIB_PATH,
    SIGNATURES,
    attn_decode_paged,
    attn_decode_paged_q8,
    attn_decode_paged_workspace_size,
    attn_dsa_indexer,
    attn_kv_append_paged,
    attn_mla_decode,
    attn_mla_decode_q8,
    attn_mla_decode_workspace_size,
    attn_mla_sparse_decode,
    attn_mla_sparse_decode_workspace_size,
    attn_prefill,
    attn_prefill_local_global,
    attn_prefill_paged,
    attn_prefill_paged_rope,
    attn_prefill_rope,
    attn_rope_apply,
    attn_rope_table,
    attn_topk,
    load_library,
)
