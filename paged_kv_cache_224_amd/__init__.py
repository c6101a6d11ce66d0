"""PagedAttention decode for AMD Instinct MI355X (gfx950).

The hot path (KV write scatter, paged decode attention, split-K log-sum-exp reduce) runs in
hand-written HIP kernels in libpagedkv.so behind a C ABI (include/pagedkv.h).  This package
is the thin ctypes binding over it plus a seeded synthetic workload generator.
"""
from ._lib import (BlockManager, DecodeWorkspace, PagedKVError, SharedPrefixWorkspace, balanced_split, decode,
                   decode_append, decode_shared_prefix, lib, multi_query, multi_query_split, paged_attn_decode, paged_attn_decode_append, paged_attn_decode_noalloc, paged_attn_decode_shared_prefix,
                   paged_attn_multi_query, paged_attn_reduce, paged_attn_workspace_bytes, paged_kv_copy_blocks,
                   paged_kv_swap_blocks, paged_kv_write, prefix_split, status_string, time_next_call)

__all__ = ["BlockManager", "DecodeWorkspace", "PagedKVError", "SharedPrefixWorkspace", "balanced_split", "decode",
           "decode_append", "decode_shared_prefix", "lib", "multi_query", "multi_query_split", "paged_attn_decode", "paged_attn_decode_append", "paged_attn_decode_noalloc", "paged_attn_decode_shared_prefix",
           "paged_attn_multi_query", "paged_attn_reduce", "paged_attn_workspace_bytes", "paged_kv_copy_blocks",
           "paged_kv_swap_blocks", "paged_kv_write", "prefix_split", "status_string", "time_next_call"]
