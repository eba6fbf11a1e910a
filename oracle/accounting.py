"""Byte and utilisation accounting (oracle).

* KV-cache size: batch x sequence length x layers x hidden width x 2 (K and V)
  x bytes per element (gheillcoat.github.io, "概念-vLLM", section
  核心概念：KV Cache 与显存效率).  With grouped KV heads the width per token is
  Hkv x head_dim rather than the model's hidden width.
* Paged utilisation: only the last block of each sequence can hold unused
  slots (explore.n1n.ai, "vLLM 深度解析", 映射机制详解), so the fraction of
  allocated slots holding tokens is sum L / (bs * sum ceil(L / bs)), bs the
  block size (16 unless stated).
* Contiguous reservation, the scheme paging replaces: every sequence reserves
  ``max_len`` slots up front (explore.n1n.ai, section on KV-cache
  fragmentation), so the used fraction is sum L / (B * max_len).
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def kv_cache_bytes(batch: int, seq_len: int, layers: int, width: int,
                   elem_bytes: int) -> int:
    return int(batch) * int(seq_len) * int(layers) * int(width) * 2 * int(elem_bytes)


def paged_utilisation(lens, block_size: int = BLOCK) -> float:
    L = np.asarray(lens, dtype=np.int64)
    slots = int(block_size) * int(np.sum(-(-L // int(block_size))))
    return float(L.sum()) / slots if slots else 1.0


def contiguous_utilisation(lens, max_len: int) -> float:
    L = np.asarray(lens, dtype=np.int64)
    return float(L.sum()) / (len(L) * int(max_len))
