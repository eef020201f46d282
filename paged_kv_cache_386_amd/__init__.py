"""libpagedattn: PagedAttention decode, KV-cache write and copy-on-write block
copy as hand-written HIP kernels for gfx950 (MI355X), behind a C ABI.

The Python names mirror the C entry points in ``include/pagedattn.h``; they
only marshal arguments (torch supplies device memory and the stream).
"""
from ._lib import (  # noqa: F401
    BlockManager,
    BlockStats,
    Engine,
    EngineConfig,
    StepInfo,
    PA_BF16,
    PA_F32,
    PA_FP8_E4M3,
    PA_ERR_INDEX,
    PA_INT8,
    PagedAttnError,
    copy_blocks,
    decode_plan,
    index_check,
    kv_cache_append,
    kv_cache_write,
    kv_cache_write_fp8,
    kv_cache_write_int8,
    lib,
    multi_query_partitions,
    multi_query_workspace_size,
    noalloc_scratch_bytes,
    num_partitions,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_decode_prefix,
    prefix_groups,
    prefix_workspace_size,
    paged_attention_decode_fp8,
    paged_attention_decode_int8,
    paged_attention_multi_query,
    paged_attention_multi_query_fp8,
    paged_attention_multi_query_int8,
    partition_tokens,
    set_index_check,
    workspace_size,
)
