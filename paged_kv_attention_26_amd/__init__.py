"""Paged attention over a block-table-indexed KV cache for AMD MI355X (gfx950).

A thin Python binding over libpa.so's C ABI (include/pa.h): argument
marshalling only.  torch provides device memory and streams; every step of
the attention path runs in libpa's HIP kernels.

Calls:
  store_kv        scatter new K/V rows into their slots
  copy_blocks     copy-on-write block copies
  decode          one query per sequence through the block table (split-K)
  prefill_chunk   causal chunk over its paged prefix (matrix cores)
  BlockManager    host block manager (allocate / fork / copy on write)
"""
from .binding import (KVCache, BlockManager, alloc_cache, store_kv, copy_blocks, decode, decode_workspace,
                      decode_workspace_bytes, prefill_chunk, DTYPE_CODES)

__all__ = ["KVCache", "BlockManager", "alloc_cache", "store_kv", "copy_blocks", "decode", "decode_workspace",
           "decode_workspace_bytes", "prefill_chunk", "DTYPE_CODES"]
