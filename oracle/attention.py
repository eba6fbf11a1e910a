"""Single-query decode attention over a paged KV cache (oracle, float64).

What is computed (the decode-time attention step of the pages): for every
sequence s and query head h, the new token's query attends over the keys and
values of all ``context_lens[s]`` cached tokens of that sequence, which live in
fixed-size blocks scattered through a physical pool and are found through the
sequence's block table.

* Blocks of 16 tokens, a per-sequence block table mapping logical block index
  to physical block: explore.n1n.ai, "vLLM 深度解析：PagedAttention 如何让大模型
  推理更快、更省钱", section 映射机制详解; ybb.press, "vLLM PagedAttention
  大模型推理架构深度实战", §2.2.
* The kernel walks ceil(len / block_size) table entries of each sequence and
  reads the blocks they name: unionyoga.cn, "vLLM：重塑大模型推理性能的关键
  引擎", section "vLLM 如何破局？从PagedAttention说起" (kernel sketch).
* Exact attention; blockwise partial results are merged with online-softmax
  renormalisation: ybb.press, §5.1.
* Query heads share KV heads (GQA/MQA): ybb.press, §9 item 3.

Readings where the pages are silent:

* Cache layout: two tensors (K and V), each ``[num_blocks, Hkv, 16, D]``;
  element (b, g, t, d) sits at ((b*Hkv + g)*16 + t)*D + d.
* Query head h reads KV head floor(h / G), G = Hq / Hkv.
* Only the first ``context_lens[s]`` positions are attended; slots past that in
  the last block are never read (so garbage there cannot leak in), and table
  entries past ceil(L / 16) are never read.
* ``context_lens[s] == 0`` gives an all-zero output row.
* Logits are ``scale * q.k`` with the caller's float32 scale widened to
  float64; no mask other than the context length.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, widen_cache

BLOCK = 16


def _q64(q: np.ndarray, q_fmt: str) -> np.ndarray:
    if q_fmt == "f32":
        return np.asarray(q, dtype=np.float32).astype(np.float64)
    if q_fmt == "bf16":
        return bf16_to_f64(q)
    raise ValueError(q_fmt)


def gather_kv(cache: np.ndarray, block_table_row: np.ndarray, L: int,
              g: int) -> np.ndarray:
    """Contiguous [L, D] rows of KV head g for one sequence, in storage format.

    Walks table entries j = 0 .. ceil(L/bs)-1 (bs = the cache's tokens per
    block, 16 unless stated), takes physical block ``block_table_row[j]``
    (all bs slots of head g), concatenates and keeps the first L rows.
    """
    bs = cache.shape[2]                          # tokens per block
    n = -(-int(L) // bs)
    if n == 0:
        return cache[:0, g, :, :].reshape(0, cache.shape[-1])
    ids = np.asarray(block_table_row[:n], dtype=np.int64)
    tiles = cache[ids, g, :, :]                  # [n, bs, D]
    return tiles.reshape(n * bs, cache.shape[-1])[:L]


def decode(q: np.ndarray, q_fmt: str, k_cache: np.ndarray, v_cache: np.ndarray,
           fmt: str, block_tables: np.ndarray, context_lens: np.ndarray,
           scale: np.float32, k_scale: float = 1.0, v_scale: float = 1.0,
           seqs=None, want_weights: bool = False):
    """Textbook softmax attention per (sequence, query head), float64.

    For s, h: g = h // G, L = context_lens[s];
    K_s, V_s = gathered rows widened to float64 (fp8: code value x scale);
    z_t = scale * sum_d q[s,h,d] K_s[t,d]; m = max_t z_t;
    w_t = exp(z_t - m) / sum_u exp(z_u - m); out[s,h] = sum_t w_t V_s[t].

    Returns ``out`` [B, Hq, D] float64 (rows of sequences not in ``seqs`` are
    NaN) and, if ``want_weights``, a dict {(s, h): w}.
    """
    q64 = _q64(q, q_fmt)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = np.float64(np.float32(scale))
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    weights = {}
    seqs = range(B) if seqs is None else seqs
    for s in seqs:
        L = int(context_lens[s])
        for g in range(Hkv):
            heads = range(g * G, (g + 1) * G)
            if L == 0:
                for h in heads:
                    out[s, h] = 0.0
                    weights[(s, h)] = np.zeros(0)
                continue
            K = widen_cache(gather_kv(k_cache, block_tables[s], L, g), fmt, k_scale)
            V = widen_cache(gather_kv(v_cache, block_tables[s], L, g), fmt, v_scale)
            for h in heads:
                z = sc * (K @ q64[s, h])
                m = z.max()
                e = np.exp(z - m)
                w = e / e.sum()
                out[s, h] = w @ V
                if want_weights:
                    weights[(s, h)] = w
    return (out, weights) if want_weights else out


def merge_partitions(m: np.ndarray, l: np.ndarray, o_hat: np.ndarray) -> np.ndarray:
    """Combine per-partition softmax results into the full-context result.

    Partition i contributes its running max m_i, its exponent sum
    l_i = sum_t exp(z_t - m_i) and its normalised output o_hat_i.  With
    M = max_i m_i:  out = sum_i exp(m_i - M) l_i o_hat_i / sum_i exp(m_i - M) l_i.
    This is the online-softmax merge of blockwise results (ybb.press, §5.1).
    """
    M = np.max(m)
    a = np.exp(m - M) * l
    return (a[:, None] * o_hat).sum(axis=0) / a.sum()


def decode_partitioned(q: np.ndarray, q_fmt: str, k_cache: np.ndarray,
                       v_cache: np.ndarray, fmt: str, block_tables: np.ndarray,
                       context_lens: np.ndarray, scale: np.float32,
                       k_scale: float = 1.0, v_scale: float = 1.0,
                       partition: int = 512, seqs=None) -> np.ndarray:
    """Same result as ``decode``, computed per ``partition``-token slice of the
    context and merged with ``merge_partitions``."""
    q64 = _q64(q, q_fmt)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = np.float64(np.float32(scale))
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    seqs = range(B) if seqs is None else seqs
    for s in seqs:
        L = int(context_lens[s])
        for g in range(Hkv):
            if L == 0:
                out[s, g * G:(g + 1) * G] = 0.0
                continue
            K = widen_cache(gather_kv(k_cache, block_tables[s], L, g), fmt, k_scale)
            V = widen_cache(gather_kv(v_cache, block_tables[s], L, g), fmt, v_scale)
            for h in range(g * G, (g + 1) * G):
                ms, ls, os_ = [], [], []
                for start in range(0, L, partition):
                    z = sc * (K[start:start + partition] @ q64[s, h])
                    mi = z.max()
                    e = np.exp(z - mi)
                    li = e.sum()
                    ms.append(mi)
                    ls.append(li)
                    os_.append((e @ V[start:start + partition]) / li)
                out[s, h] = merge_partitions(np.array(ms), np.array(ls), np.array(os_))
    return out
