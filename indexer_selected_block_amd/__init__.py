"""Indexed block-sparse paged-attention decode for AMD Instinct MI355X (gfx950).

The compute lives in libisb.so (hand-written HIP kernels behind a C ABI,
declared in include/isb.h); ``binding`` marshals torch tensors into it and
``workload`` builds seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    DecodeLayer,
    PrefillLayer,
    IsbError,
    emit_sparse_block_table,
    emit_sparse_block_table_prefill,
    index_score,
    index_score_prefill,
    NormRope,
    load_library,
    norm_rope,
    prepare_query,
    quantize_e4m3,
    select_attend,
    select_attend_prefill,
    sparse_pa_decode,
    sparse_pa_decode_noalloc,
    sparse_pa_prefill,
    sparse_pa_workspace_bytes,
    strerror,
    topk_select,
    topk_select_prefill,
    topk_merge,
    topk_select_emit,
    topk_select_emit_prefill,
    version,
    write_cache,
    write_cache_launcher,
)
