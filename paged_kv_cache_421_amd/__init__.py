"""Paged KV cache and single-query decode attention for AMD Instinct MI355X.

Python binding of libpagedkv (include/pagedkv.h).  Every function only
marshals arguments -- torch tensors to device pointers, the current HIP stream
-- and calls the C ABI; all device work runs in the library's gfx950 kernels.
"""
from __future__ import annotations

from ._lib import LIB_PATH, PagedKVError, lib
from .api import (BLOCK_SIZE, MAX_CHUNK, PARTITION_TOKENS, BlockManager, CacheDesc,
                  chunk_workspace_bytes, copy_blocks, decode, decode_chunk, decode_noalloc,
                  decode_workspace_bytes, decode_workspace_init, dtype_code,
                  new_chunk_workspace, new_decode_workspace, read_probe, swap_blocks, write_kv,
                  decode_shared_prefix, new_shared_prefix_workspace,
                  shared_prefix_workspace_bytes, time_next_call)

__all__ = ["LIB_PATH", "PagedKVError", "lib", "BLOCK_SIZE", "MAX_CHUNK", "PARTITION_TOKENS",
           "BlockManager", "CacheDesc", "chunk_workspace_bytes", "copy_blocks", "decode",
           "decode_chunk", "decode_noalloc", "decode_workspace_bytes", "decode_workspace_init", "dtype_code",
           "new_chunk_workspace", "new_decode_workspace", "read_probe", "swap_blocks", "write_kv",
           "decode_shared_prefix", "new_shared_prefix_workspace",
           "shared_prefix_workspace_bytes", "time_next_call"]
