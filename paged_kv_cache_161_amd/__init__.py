"""MI355X (gfx950) PagedAttention: paged KV append, paged decode, paged (chunked)
prefill, block copies for copy-on-write and a host block allocator.

The computation runs in the HIP library libpa_mi355x.so (C ABI in
include/paged_attention.h); `binding` marshals torch tensors into it.
`workloads` builds seeded synthetic inputs and holds no attention arithmetic.
"""
from .binding import (BLOCK_SIZE, BlockAllocator, PaError, cache_append, copy_blocks, decode,
                      decode_append, load, partition_tokens, pool_bytes, prefill, workspace_bytes)

__all__ = ["BLOCK_SIZE", "BlockAllocator", "PaError", "cache_append", "copy_blocks", "decode",
           "decode_append", "load", "partition_tokens", "pool_bytes", "prefill", "workspace_bytes"]
