"""Paged decode attention for AMD Instinct MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels behind a C ABI,
declared in include/pa.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PA_KV_FP16,
    PA_KV_FP8_E4M3,
    BlockManager,
    BlockManagerError,
    copy_blocks,
    pa_copy_blocks,
    PagedAttentionError,
    exported_symbols,
    kv_dtype_of,
    load_library,
    pa_abi_version,
    pa_decode_v1,
    pa_decode_v2,
    pa_decode_v2_shared,
    pa_decode_v2_noalloc,
    pa_prefill,
    pa_gather_kv,
    pa_reduce,
    pa_v2_max_partitions,
    paged_attention_v1,
    paged_attention_v2,
    reshape_and_cache,
    pa_reshape_and_cache,
    split_kv_cache,
    v2_scratch,
)
