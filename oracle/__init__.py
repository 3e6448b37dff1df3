"""fp64 CPU oracle for exact attention with RoPE — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import this
package. The product path (the HIP library and its Python binding) never imports, links or calls it, and it
shares no code with that path: it is written from the pages' definitions, in plain numpy float64.

Every function here is pinned by ``tests/test_oracle_pins.py`` to something other than itself (closed forms,
brute force, invariants, a library routine in a special case). No function is "parity unpinned".
"""
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    rope_inv_freq,
    rope,
    attention_prefill,
    attention_prefill_rows,
    gather_paged,
    decode_paged,
    mla_decode,
    mla_naive,
    kv_append_paged,
    prefill_paged,
    dsa_indexer_scores,
    topk_indices,
    mla_sparse_decode,
    fp8_e4m3_decode,
    int8_decode,
    dequantize_kv,
    decode_paged_q8,
    local_global_visible,
    attention_local_global,
    mla_decode_q8,
    attention_local_global_rows,
)
