"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The hot path is a C-ABI library (libpa.so, hand-written HIP kernels, declared
in include/pa.h); this package is its thin Python binding:

    cache_write(kv_pool, key, value, block_tables, context_lens, k_scale, v_scale)
    decode(query, kv_pool, block_tables, context_lens, scale, k_scale, v_scale, ...)
    decode_noalloc(query, kv_pool, block_tables, context_lens, scale, k_scale, v_scale, out=...)
    cache_write_tokens(kv_pool, key, value, block_tables, context_lens, cu_seqlens, k_scale, v_scale)
    prefill(query, kv_pool, block_tables, context_lens, cu_seqlens, scale, k_scale, v_scale)
    copy_blocks(src_pool, dst_pool, block_mapping)

Build the library with ``python -m paged_kv_cache_132_amd.build``.
"""
from ._lib import (
    PA_BF16,
    PA_F16,
    PA_FP8_E4M3,
    EXPORTED,
    LIB_PATH,
    Workspace,
    cache_write,
    cache_write_tokens,
    copy_blocks,
    decode,
    decode_noalloc,
    decode_partition_size,
    decode_workspace_size,
    load,
    pa_dtype,
    prefill,
)

__all__ = [
    "PA_F16", "PA_BF16", "PA_FP8_E4M3", "EXPORTED", "LIB_PATH", "Workspace", "cache_write", "cache_write_tokens", "copy_blocks", "decode",
    "decode_noalloc", "decode_partition_size", "decode_workspace_size", "load", "pa_dtype", "prefill",
]
