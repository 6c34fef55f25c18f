"""CPU oracle for paged, variable-length attention over a page-table-indexed KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``paged_kv_cache_197_amd``) never imports it and shares no code,
header, table or helper with it.

Everything here is plain, slow float64 numpy written from the pages below; every
function names the passage it follows. Pages are cited by title and section
(the function or class on that page):

  [DCA] "sglang 0.4.10.post2 -> 0.5.0rc0: sglang/srt/layers/attention/
         dual_chunk_flashattention_backend.py"
  [XPU] "sglang 0.5.3rc2 -> 0.5.4: sglang/srt/layers/attention/xpu_backend.py"
  [FA]  "sgl-project--sglang/python/sglang/srt/layers/attention/
         flashattention_backend.py"
  [NSA] "sglang/srt/layers/attention/nsa_backend.py"

Pin status: every function is pinned by a CPU test (closed forms, the pages'
worked examples under tests/golden/, a library routine on special cases, or
brute force). Attention *values* have no printed example on the pages; their
pins are the closed forms and the library/brute-force special cases.
"""

from .reference import (  # noqa: F401
    NEG_INF,
    cascade_attention,
    cascade_expand_table,
    causal_key_ranges,
    cu_seqlens,
    dca_decode,
    dca_decode_reference,
    dca_decode_tables,
    dca_query_chunk,
    dca_scaling_factor,
    gather_paged,
    key_lower_bound,
    kv_append,
    local_attention_virtual_batches,
    kv_head_of,
    merge_state,
    page_table_pa_swa,
    page_table_strided,
    paged_decode_splitkv,
    paged_prefill,
    paged_prefill_append,
    round_to_bf16,
    softmax_attention,
    sparse_topk_decode,
    tree_verify_attention,
    visible_key_counts,
)
