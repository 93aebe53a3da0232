"""MI355X (gfx950) paged attention over a block-table KV cache.

Python binding of libpagedattn.so (C ABI in include/pagedattn.h).  The
functions below only check and marshal torch tensors into pointers and sizes;
every step of the computation runs in the library's HIP kernels.  There is no
CPU fallback: a call fails if the library is not built or the tensors are
not on a GPU.
"""
from .ops import (  # noqa: F401
    LAYOUT_MLA_LATENT,
    LAYOUT_SHUFFLED_KV,
    LAYOUT_STANDARD_KV,
    NOALLOC_SCRATCH_BYTES,
    PagedAttnError,
    PreparedCall,
    WORKSPACE_COUNTER_BYTES,
    chunked_extend_attn,
    decode_partition_tokens,
    decode_uses_balanced_split,
    decode_workspace_size,
    extend_chunk_tokens,
    extend_workspace_size,
    gather_cache_chunk,
    gather_cache_chunk_fp8,
    library,
    merge_attn_states,
    mla_decode_attn,
    mla_decode_attn_mfma,
    mla_decode_attn_write,
    mixed_batch_attn,
    mixed_batch_plan,
    mla_workspace_size,
    paged_decode_attn,
    paged_decode_attn_fp8,
    mla_decode_attn_fp8,
    mla_decode_attn_fp8_mfma,
    paged_decode_attn_layout,
    paged_decode_attn_write,
    paged_decode_attn_write_noalloc,
    prepare,
    reshape_and_cache,
    reshape_and_cache_fp8,
    reshape_and_cache_mla_fp8,
    stream_read,
    gather_read,
)
