"""Writes into and copies within the paged KV cache (oracle, bit-exact).

* ``write_kv``: after attention, each decode iteration stores the new token's
  K and V into its sequence's current block (ybb.press, "vLLM PagedAttention
  大模型推理架构深度实战", §6 decode loop).  The destination of token i is given
  as a flat slot number ``slot_mapping[i]`` = physical block * block_size + offset
  (reading: the pages fix no form; a negative slot means "skip this row").
* ``copy_blocks``: copy-on-write duplicates a shared block before a sequence
  modifies it (ybb.press, §2.3).  Every (src, dst) pair copies the whole
  block -- all KV heads, all slots -- of both caches, byte for byte.
  Precondition (reading): destinations are distinct and no destination is also
  a source, so the pairs commute.
* ``swap_blocks``: the same whole-block copies between two pools, the device
  cache and a host pool, for swapping sequences out and back in.

Caches are ``[num_blocks, Hkv, block_size, D]`` arrays (block_size 16 unless stated) in storage format (float32,
uint16 bf16 bits, or uint8 E4M3 codes).  Both functions return new arrays and
leave every byte they do not write untouched.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_encode

BLOCK = 16


def _convert(rows: np.ndarray, src_fmt: str, fmt: str, scale) -> np.ndarray:
    if src_fmt == fmt:
        return rows                                      # identical bits
    if src_fmt == "bf16" and fmt == "fp8":
        x = (np.asarray(rows, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        inv = np.float32(1.0 / np.float64(np.float32(scale)))   # correctly rounded fp32(1/scale)
        return e4m3_encode(x, inv)
    raise ValueError(f"unsupported conversion {src_fmt} -> {fmt}")


def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray,
             v: np.ndarray, slot_mapping: np.ndarray, src_fmt: str, fmt: str,
             k_scale: float = 1.0, v_scale: float = 1.0):
    """Scatter rows ``k[i], v[i]`` ([Hkv, D] each) into slot ``slot_mapping[i]``.

    For slot >= 0: block = slot // bs, offset = slot % bs (bs = the cache's
    tokens per block, 16 unless stated), and for every KV head g:
    cache[block, g, offset, :] = convert(row[g, :]).  Returns the new
    (k_cache, v_cache).
    """
    kc = k_cache.copy()
    vc = v_cache.copy()
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    bs = k_cache.shape[2]                        # tokens per block
    blk = slots[keep] // bs
    off = slots[keep] % bs
    kc[blk, :, off, :] = _convert(np.asarray(k)[keep], src_fmt, fmt, k_scale)
    vc[blk, :, off, :] = _convert(np.asarray(v)[keep], src_fmt, fmt, v_scale)
    return kc, vc


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> tuple:
    """For each (src, dst): K[dst] = K[src] and V[dst] = V[src] (whole blocks)."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
    return kc, vc


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                pairs) -> tuple:
    """Block copies between two pools (device cache and host pool, either way):
    for each (s, d), dst[d] = src[s] for both caches, whole blocks, byte for
    byte (ybb.press §3.2: a swapped-out sequence's KV moves to CPU memory and
    back).  Returns new destination arrays; the sources are unchanged."""
    kd = dst_k.copy()
    vd = dst_v.copy()
    for s, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        kd[d] = src_k[s]
        vd[d] = src_v[s]
    return kd, vd
