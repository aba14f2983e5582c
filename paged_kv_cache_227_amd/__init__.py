"""MI355X-native paged KV cache decode path.

The compute path is the HIP library libpagedkv.so (C ABI in include/pagedkv.h);
this package binds it (``_lib``), and holds the host block manager
(``blocks``) and the seeded input generator (``workloads``).
"""
from ._lib import (NOALLOC_SCRATCH_BYTES, PagedKVCache, alloc_workspace, last_error, layout_of,
                   paged_attention_decode, paged_attention_decode_noalloc,
                   paged_attention_merge, paged_attention_partitions, paged_kv_append,
                   paged_kv_append_attention_decode,
                   paged_kv_copy_blocks, validate_copies, paged_kv_append_tokens,
                   paged_attention_prefill, validate_prefill, paged_kv_swap_out, paged_kv_swap_in,
                   partition_tokens_for, probe_copy, probe_read, set_partition_tokens, validate,
                   version, workspace_size)

__all__ = ["NOALLOC_SCRATCH_BYTES", "PagedKVCache", "alloc_workspace", "last_error", "layout_of",
           "paged_attention_decode", "paged_attention_decode_noalloc",
           "paged_attention_merge", "paged_attention_partitions", "paged_kv_append",
           "paged_kv_append_attention_decode", "paged_kv_copy_blocks",
           "validate_copies", "paged_kv_append_tokens", "paged_attention_prefill", "validate_prefill",
           "paged_kv_swap_out", "paged_kv_swap_in",
           "partition_tokens_for", "probe_copy", "probe_read", "set_partition_tokens", "validate",
           "version", "workspace_size"]
