"""Attention of a chunk of new query tokens over a paged KV cache (oracle,
float64) -- TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``.

What is computed: a step that brings T > 1 new tokens of a sequence at once,
as when a long prompt is fed in chunks (chunked prefill, ybb.press, "vLLM
PagedAttention 大模型推理架构深度实战", §7.1 and §7.2) or when the target model
checks several draft tokens in one pass (speculative decoding, same page, §9
item 2).  The chunk's K and V rows have been written into the paged cache
first, as in single-token decode (same page, §6: write KV, then attend), so
``context_lens[s] = L`` counts them.  Each new token attends exactly as it
would in its own decode step.

Reading where the pages are silent (plainest reading, causal order):

* chunk token i (0 <= i < T) of sequence s sits at position L - T + i and
  attends positions 0 .. L - T + i of that sequence (itself and every earlier
  token, never a later chunk token);
* a token with no visible position (L - T + i < 0, i.e. L < T - i) gets a zero
  output row, the rule for an empty context;
* q and out are ``[B, T, Hq, D]``; every other convention (layout, GQA head
  map, scale, fp8 scales) is the single-token decode's.

Sliding window (ybb.press §7.2: for long contexts, enable sliding-window
attention).  Reading: with a window of W > 0 positions, a token at position
p attends only the last W positions up to itself, max(0, p - W + 1) .. p;
W = 0 means no window.  Windowed single-token decode is T = 1.
"""
from __future__ import annotations

import numpy as np

from .attention import _q64, gather_kv
from .formats import widen_cache


def visible_len(L: int, T: int, i: int) -> int:
    """Positions chunk token i of a length-L context may attend (its own
    position + 1): 0 .. L - T + i."""
    return max(0, int(L) - int(T) + int(i) + 1)


def window_start(n: int, window: int) -> int:
    """First attended position when the last one is n - 1."""
    return max(0, int(n) - int(window)) if window > 0 else 0


def decode_chunk(q: np.ndarray, q_fmt: str, k_cache: np.ndarray, v_cache: np.ndarray,
                 fmt: str, block_tables: np.ndarray, context_lens: np.ndarray,
                 scale: np.float32, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs=None, window: int = 0) -> np.ndarray:
    """Textbook softmax attention per (sequence, chunk token, query head).

    For s, i, h: g = h // G, n = L - T + i + 1, a = window_start(n, window);
    K, V = gathered rows a .. n-1 of KV head g, widened to float64;
    z_t = scale * q[s,i,h] . K[t]; w = softmax(z); out[s,i,h] = w @ V
    (zero if n == 0).  Rows of sequences not in ``seqs`` are NaN.
    """
    q64 = _q64(q, q_fmt)
    B, T, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = np.float64(np.float32(scale))
    out = np.full((B, T, Hq, D), np.nan, dtype=np.float64)
    seqs = range(B) if seqs is None else seqs
    for s in seqs:
        L = int(context_lens[s])
        for g in range(Hkv):
            K = widen_cache(gather_kv(k_cache, block_tables[s], L, g), fmt, k_scale)
            V = widen_cache(gather_kv(v_cache, block_tables[s], L, g), fmt, v_scale)
            for i in range(T):
                n = visible_len(L, T, i)
                a = window_start(n, window)
                for h in range(g * G, (g + 1) * G):
                    if n == 0:
                        out[s, i, h] = 0.0
                        continue
                    z = sc * (K[a:n] @ q64[s, i, h])
                    e = np.exp(z - z.max())
                    out[s, i, h] = (e / e.sum()) @ V[a:n]
    return out


def chunk_rows(q: np.ndarray, q_fmt: str, k_cache, v_cache, fmt, block_tables,
               context_lens, scale, k_scale=1.0, v_scale=1.0, picks=(), window: int = 0) -> np.ndarray:
    """``decode_chunk`` for a sample of (sequence, chunk token, query head)
    triples only: [len(picks), D] float64."""
    q64 = _q64(q, q_fmt)
    B, T, Hq, D = q64.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    sc = np.float64(np.float32(scale))
    rows = []
    for (s, i, h) in picks:
        L = int(context_lens[s])
        n = visible_len(L, T, i)
        if n == 0:
            rows.append(np.zeros(D))
            continue
        g = h // G
        a = window_start(n, window)
        K = widen_cache(gather_kv(k_cache, block_tables[s], n, g), fmt, k_scale)[a:]
        V = widen_cache(gather_kv(v_cache, block_tables[s], n, g), fmt, v_scale)[a:]
        z = sc * (K @ q64[s, i, h])
        e = np.exp(z - z.max())
        rows.append((e / e.sum()) @ V)
    return np.array(rows).reshape(len(picks), D)
