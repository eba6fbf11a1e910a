"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the paged
decode path computes, in float64 wherever floating point is involved.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library (no
kernels, headers, helpers or constant tables) and never imports it; the two
meet only at the seeded arrays produced by ``workloads``.

Sources (all web pages on vLLM / PagedAttention):

* explore.n1n.ai, "vLLM 深度解析：PagedAttention 如何让大模型推理更快、更省钱"
* ybb.press, "vLLM PagedAttention 大模型推理架构深度实战"
* unionyoga.cn, "vLLM：重塑大模型推理性能的关键引擎"
* gheillcoat.github.io, "概念-vLLM"

Each function cites the section it follows.  Every function is pinned by a
``-m "not gpu"`` test to something other than itself (brute force, closed
forms, invariants, a library routine); none is "parity unpinned".
"""
from .formats import (bf16_to_f64, e4m3_to_f64, e4m3_encode, e4m3_all_values,
                      widen_cache)
from .attention import gather_kv, decode, decode_partitioned, merge_partitions
from .chunk import decode_chunk, chunk_rows, visible_len
from .cache_ops import write_kv, copy_blocks, swap_blocks
from .block_manager import RefBlockManager, NoBlocks, UnknownSeq, SeqExists, Swapped, block_key
from .accounting import kv_cache_bytes, paged_utilisation, contiguous_utilisation

__all__ = [
    "bf16_to_f64", "e4m3_to_f64", "e4m3_encode", "e4m3_all_values", "widen_cache",
    "gather_kv", "decode", "decode_partitioned", "merge_partitions",
    "decode_chunk", "chunk_rows", "visible_len",
    "write_kv", "copy_blocks", "swap_blocks",
    "RefBlockManager", "NoBlocks", "UnknownSeq", "SeqExists", "Swapped", "block_key",
    "kv_cache_bytes", "paged_utilisation", "contiguous_utilisation",
]
