"""Paged-KV attention for AMD Instinct MI355X (gfx950).

Python binding of libpagedkv, whose C ABI is ``include/pagedkv.h``:

* ``kv_cache_write``  -- store new K/V vectors in physical block slots
  (bf16/fp32 copy, or INT8 with a dynamic per-vector fp16 scale);
* ``paged_attention_decode`` -- one query token per sequence, split over
  partitions of the context and merged (log-sum-exp);
* ``paged_attention_prefill_chunk`` -- a chunk of query tokens per sequence
  with causal and sliding-window masks, on bf16 MFMA;
* ``build_slot_mapping`` / ``kv_cache_copy_blocks`` -- slots of a step's new
  rows from the block tables, and whole-block copies (copy on write), on the GPU;
* ``BlockAllocator`` -- host-side block ownership: O(1) free stack, reference
  counts for shared prefixes, append / fork / rollback / window eviction.

The library is loaded on first use; there is no CPU fallback.
"""
from ._binding import (EXPORTS, LIB_PATH, BlockAllocator, CacheDesc, PagedKVError, build_slot_mapping,
                       cache_desc, decode_workspace, decode_workspace_size, kv_cache_copy_blocks, kv_cache_write, last_error,
                       load_library, paged_attention_decode, paged_attention_decode_noalloc,
                       decode_noalloc_max_scratch, paged_attention_prefill_chunk,
                       set_decode_split_event, set_decode_start_event, version)

__all__ = ["EXPORTS", "LIB_PATH", "BlockAllocator", "CacheDesc", "build_slot_mapping", "kv_cache_copy_blocks", "PagedKVError", "cache_desc", "decode_workspace", "decode_workspace_size",
           "kv_cache_write", "last_error", "load_library", "paged_attention_decode", "paged_attention_decode_noalloc", "decode_noalloc_max_scratch",
           "paged_attention_prefill_chunk", "set_decode_split_event", "set_decode_start_event", "version"]
