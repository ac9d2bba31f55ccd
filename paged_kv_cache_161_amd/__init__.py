"""MI355X (gfx950) decode-phase PagedAttention: paged KV append and paged decode.

The computation runs in the HIP library libpa_mi355x.so (C ABI in
include/paged_attention.h); `binding` marshals torch tensors into it.
`workloads` builds seeded synthetic inputs and holds no attention arithmetic.
"""
from .binding import (BLOCK_SIZE, PaError, cache_append, decode, load, partition_tokens,
                      pool_bytes, workspace_bytes)

__all__ = ["BLOCK_SIZE", "PaError", "cache_append", "decode", "load", "partition_tokens",
           "pool_bytes", "workspace_bytes"]
