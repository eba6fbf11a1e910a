"""Paged KV cache and single-query decode attention for AMD Instinct MI355X.

Python binding of libpagedkv (include/pagedkv.h).  Every function only
marshals arguments -- torch tensors to device pointers, the current HIP stream
-- and calls the C ABI; all device work runs in the library's gfx950 kernels.
"""
from __future__ import annotations

from ._lib import LIB_PATH, PagedKVError, lib
from .api import (BLOCK_SIZE, PARTITION_TOKENS, BlockManager, CacheDesc, copy_blocks,
                  decode, decode_workspace_bytes, decode_workspace_init, dtype_code,
                  new_decode_workspace, write_kv)

__all__ = ["LIB_PATH", "PagedKVError", "lib", "BLOCK_SIZE", "PARTITION_TOKENS",
           "BlockManager", "CacheDesc", "copy_blocks", "decode",
           "decode_workspace_bytes", "decode_workspace_init", "dtype_code",
           "new_decode_workspace", "write_kv"]
