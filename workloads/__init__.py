"""Seeded synthetic inputs for the paged decode-attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, no block allocation, no quantisation).  Both
the GPU path and the CPU oracle receive exactly the arrays produced here, so a
test can feed identical inputs to two independent implementations.

Five workloads are defined, each with its own ``numpy.random.default_rng(seed)``
(seed = workload number).  Draw order inside a workload is fixed:

1. random context lengths (and, for the copy-on-write workload, the fork
   offsets ``r`` and then the suffix lengths);
2. the physical-block permutation handed to the block manager as its free
   order;
3. K rows for every token, in (sequence, position) order (copy-on-write
   workload: per group the shared prefix rows once, then each sample's suffix);
4. V rows, the same way;
5. q ``[B, Hq, D]``.

Floating-point rows are drawn in float32 (``uniform(-1, 1)`` or
``standard_normal``) and, for 16-bit workloads, rounded to bfloat16 with
round-to-nearest-even; bfloat16 values travel as their uint16 bit patterns.

The shapes mirror the decode workloads the pages discuss: a 13B-class MHA
layer, an 8B-class GQA layer at batch 256, a 70B-class GQA layer at 32K
context, and parallel sampling with a shared prompt (ybb.press, "vLLM
PagedAttention 大模型推理架构深度实战", §2.3 and §7.2).  No dataset is read;
chat-length traces are stood in for by uniform and lognormal length draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

BLOCK = 16
PARTITION_TOKENS = 512


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even) and return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One seeded decode batch.

    ``fmt`` is the cache storage format: ``"f32"``, ``"bf16"`` or ``"fp8"``.
    ``q_fmt`` is the query/output format: ``"f32"`` or ``"bf16"``.
    ``k_rows``/``v_rows`` hold the rows to be written, in source format
    (float32, or uint16 bfloat16 bits), in the order described in the module
    docstring; ``row_seq``/``row_pos`` say which sequence and position each row
    belongs to.
    """
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    fmt: str
    q_fmt: str
    lens: np.ndarray             # int32 [B] final context lengths
    num_blocks: int              # physical pool size
    free_order: np.ndarray       # int32 [num_blocks] permutation
    k_rows: np.ndarray           # [T, Hkv, D] source rows
    v_rows: np.ndarray
    row_seq: np.ndarray          # int64 [T]
    row_pos: np.ndarray          # int64 [T]
    q: np.ndarray                # [B, Hq, D] (float32 or uint16 bits)
    scale: np.float32
    k_scale: np.float32 = np.float32(1.0)
    v_scale: np.float32 = np.float32(1.0)
    # copy-on-write workload only
    groups: Optional[List[Dict]] = None

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def src_fmt(self) -> str:
        return "f32" if self.fmt == "f32" else "bf16"

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode call reads: every valid element once."""
        e = {"f32": 4, "bf16": 2, "fp8": 1}[self.fmt]
        return int(self.lens.astype(np.int64).sum()) * self.Hkv * self.D * e * 2


def _rows(rng, shape, dist, bf16):
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    else:
        x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if bf16 else x


def _pool(lens, factor=1.25, extra=0):
    need = int(sum(-(-int(L) // BLOCK) for L in lens))
    return int(math.ceil(factor * need)) + extra


def _shape_only(name, seed, B, Hq, Hkv, D, lens, nb, perm, fmt="bf16"):
    """Lengths and pool permutation only (rows are drawn after these)."""
    return Workload(name, seed, B, Hq, Hkv, D, fmt, "bf16", lens, nb, perm,
                    None, None, None, None, None, np.float32(1.0 / math.sqrt(D)))


def _seq_rows(rng, lens, Hkv, D, dist, bf16):
    T = int(np.sum(lens))
    k = _rows(rng, (T, Hkv, D), dist, bf16)
    v = _rows(rng, (T, Hkv, D), dist, bf16)
    row_seq = np.repeat(np.arange(len(lens), dtype=np.int64), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    row_pos = np.arange(T, dtype=np.int64) - np.repeat(starts, lens)
    return k, v, row_seq, row_pos


def config1(seed: int = 1) -> Workload:
    """Tiny fp32 MHA decode: lengths {1, 15, 16, 37}, 2 heads, head_dim 64,
    a 32-block pool, uniform(-1, 1) data, scale 1/sqrt(64)."""
    rng = np.random.default_rng(seed)
    lens = np.array([1, 15, 16, 37], dtype=np.int32)
    B, H, D = 4, 2, 64
    nb = 32
    perm = rng.permutation(nb).astype(np.int32)
    k, v, rs, rp = _seq_rows(rng, lens, H, D, "uniform", False)
    q = rng.uniform(-1.0, 1.0, size=(B, H, D)).astype(np.float32)
    return Workload("tiny-mha-fp32", seed, B, H, H, D, "f32", "f32", lens, nb,
                    perm, k, v, rs, rp, q, np.float32(0.125))


def config2(seed: int = 2, rows: bool = True) -> Workload:
    """13B-shaped MHA layer, bf16: batch 64, 40 heads, head_dim 128,
    lengths uniform in [128, 2048], pool 1.25x the blocks needed."""
    rng = np.random.default_rng(seed)
    B, H, D = 64, 40, 128
    lens = rng.integers(128, 2049, B).astype(np.int32)
    nb = _pool(lens)
    perm = rng.permutation(nb).astype(np.int32)
    if not rows:
        return _shape_only("mha13b-bf16-b64", seed, B, H, H, D, lens, nb, perm)
    k, v, rs, rp = _seq_rows(rng, lens, H, D, "normal", True)
    q = _rows(rng, (B, H, D), "normal", True)
    return Workload("mha13b-bf16-b64", seed, B, H, H, D, "bf16", "bf16", lens,
                    nb, perm, k, v, rs, rp, q, np.float32(1.0 / math.sqrt(128)))


def lognormal_lens(rng, B, median=512, sigma=0.8, lo=16, hi=4096) -> np.ndarray:
    """clip(rint(exp(ln median + sigma * z)), lo, hi) with z standard normal."""
    z = rng.standard_normal(B)
    return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), lo, hi).astype(np.int32)


# Extra blocks kept free in the GQA batch-256 pool so that a decode loop can
# append up to this many tokens per sequence without running dry.
CONFIG3_MAX_APPEND = 256


def config3(seed: int = 3, rows: bool = True) -> Workload:
    """8B-shaped GQA layer, bf16: batch 256, 32 query / 8 KV heads,
    head_dim 128, lognormal lengths (median 512, sigma 0.8) in [16, 4096]."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D = 256, 32, 8, 128
    lens = lognormal_lens(rng, B)
    nb = _pool(lens, extra=B * (CONFIG3_MAX_APPEND // BLOCK + 1))
    perm = rng.permutation(nb).astype(np.int32)
    if not rows:
        return _shape_only("gqa8b-bf16-b256", seed, B, Hq, Hkv, D, lens, nb, perm)
    k, v, rs, rp = _seq_rows(rng, lens, Hkv, D, "normal", True)
    q = _rows(rng, (B, Hq, D), "normal", True)
    return Workload("gqa8b-bf16-b256", seed, B, Hq, Hkv, D, "bf16", "bf16", lens,
                    nb, perm, k, v, rs, rp, q, np.float32(1.0 / math.sqrt(128)))


def config3_step(rng: np.random.Generator, B=256, Hq=32, Hkv=8, D=128):
    """Per-iteration draws of the GQA batch-256 decode loop: k_new, v_new, q."""
    k = _rows(rng, (B, Hkv, D), "normal", True)
    v = _rows(rng, (B, Hkv, D), "normal", True)
    q = _rows(rng, (B, Hq, D), "normal", True)
    return k, v, q


def chunk_queries(rng: np.random.Generator, B: int, T: int, Hq: int, D: int,
                  fmt: str = "bf16") -> np.ndarray:
    """Queries of a chunk of T new tokens per sequence, [B, T, Hq, D]
    (uniform(-1, 1) float32 for fp32 workloads, N(0, 1) bf16 bits otherwise)."""
    if fmt == "f32":
        return _rows(rng, (B, T, Hq, D), "uniform", False)
    return _rows(rng, (B, T, Hq, D), "normal", True)


def config3_chunk_step(rng: np.random.Generator, T: int, B=256, Hq=32, Hkv=8, D=128):
    """Per-iteration draws of the GQA batch-256 loop when each step brings T
    new tokens per sequence (chunked prefill or draft verification): the
    chunk's K and V rows [B, T, Hkv, D], then its queries [B, T, Hq, D]."""
    k = _rows(rng, (B, T, Hkv, D), "normal", True)
    v = _rows(rng, (B, T, Hkv, D), "normal", True)
    q = _rows(rng, (B, T, Hq, D), "normal", True)
    return k, v, q


def config4(seed: int = 4, rows: bool = True) -> Workload:
    """70B-shaped long-context GQA layer, bf16: batch 8, 64 query / 8 KV heads,
    head_dim 128, every context 32768 tokens (2048 blocks, shuffled)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D = 8, 64, 8, 128
    lens = np.full(B, 32768, dtype=np.int32)
    nb = _pool(lens)
    perm = rng.permutation(nb).astype(np.int32)
    if not rows:
        return _shape_only("gqa70b-bf16-32k", seed, B, Hq, Hkv, D, lens, nb, perm)
    k, v, rs, rp = _seq_rows(rng, lens, Hkv, D, "normal", True)
    q = _rows(rng, (B, Hq, D), "normal", True)
    return Workload("gqa70b-bf16-32k", seed, B, Hq, Hkv, D, "bf16", "bf16", lens,
                    nb, perm, k, v, rs, rp, q, np.float32(1.0 / math.sqrt(128)))


def config5(seed: int = 5, prefix: int = 1024, aligned: bool = False,
            rows: bool = True) -> Workload:
    """Parallel sampling with a shared prompt, fp8-e4m3 cache: 64 groups x 4
    samples, 32 query / 8 KV heads, head_dim 128.

    Each group's prompt is ``prefix + r`` tokens with ``r`` uniform in [1, 15]
    (``aligned=True`` sets r = 0), so the prompt's last block is partial and
    shared by all four samples; each sample then appends a suffix of uniform
    length in [1, 256].  Rows are bf16; the fp8 scales are one per tensor,
    ``fp32(max|x| / 448)`` over every K (resp. V) value that will be stored.

    ``groups[g]`` holds ``seqs`` (4 sequence ids, parent first), ``prompt``
    (prompt length) and ``suffix`` (4 suffix lengths).  Rows are ordered per
    group: prompt rows, then each sample's suffix rows in sample order.
    """
    rng = np.random.default_rng(seed)
    NG, S, Hq, Hkv, D = 64, 4, 32, 8, 128
    B = NG * S
    r = rng.integers(1, 16, NG)
    if aligned:
        r = np.zeros(NG, dtype=np.int64)
    suf = rng.integers(1, 257, B)
    lens = np.empty(B, dtype=np.int32)
    groups = []
    for g in range(NG):
        p = prefix + int(r[g])
        seqs = [g * S + i for i in range(S)]
        sl = [int(suf[g * S + i]) for i in range(S)]
        for i in range(S):
            lens[seqs[i]] = p + sl[i]
        groups.append({"seqs": seqs, "prompt": p, "suffix": sl})
    # physical blocks: the shared prompt once per group, plus per sample the
    # blocks past the prompt and (for a partial shared block) one private copy
    need = 0
    for grp in groups:
        p = grp["prompt"]
        pb = -(-p // BLOCK)
        need += pb
        for sl in grp["suffix"]:
            need += -(-(p + sl) // BLOCK) - pb + (1 if p % BLOCK else 0)
    nb = int(math.ceil(1.25 * need))
    perm = rng.permutation(nb).astype(np.int32)
    if not rows:
        w = _shape_only("cow-fp8-4x64", seed, B, Hq, Hkv, D, lens, nb, perm, fmt="fp8")
        w.groups = groups
        return w

    def draw_rows():
        out, seq, pos = [], [], []
        for grp in groups:
            p = grp["prompt"]
            out.append(rng.standard_normal((p, Hkv, D), dtype=np.float32))
            seq.append(np.full(p, grp["seqs"][0], dtype=np.int64))
            pos.append(np.arange(p, dtype=np.int64))
            for sid, sl in zip(grp["seqs"], grp["suffix"]):
                out.append(rng.standard_normal((sl, Hkv, D), dtype=np.float32))
                seq.append(np.full(sl, sid, dtype=np.int64))
                pos.append(np.arange(p, p + sl, dtype=np.int64))
        return (f32_to_bf16_bits(np.concatenate(out)), np.concatenate(seq),
                np.concatenate(pos))

    k, rs, rp = draw_rows()
    v, _, _ = draw_rows()
    q = _rows(rng, (B, Hq, D), "normal", True)
    k_scale = np.float32(np.abs(bf16_bits_to_f32(k)).max() / np.float32(448.0))
    v_scale = np.float32(np.abs(bf16_bits_to_f32(v)).max() / np.float32(448.0))
    return Workload("cow-fp8-4x64", seed, B, Hq, Hkv, D, "fp8", "bf16", lens,
                    nb, perm, k, v, rs, rp, q, np.float32(1.0 / math.sqrt(128)),
                    k_scale, v_scale, groups)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def small_random(seed: int, B: int, Hq: int, Hkv: int, D: int, fmt: str,
                 max_len: int, min_len: int = 0, pool_factor: float = 1.5,
                 lens: Optional[np.ndarray] = None) -> Workload:
    """A small seeded batch with ragged lengths for element-wise parity tests."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(min_len, max_len + 1, B).astype(np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    nb = max(_pool(lens, pool_factor), 1)
    perm = rng.permutation(nb).astype(np.int32)
    bf16 = fmt != "f32"
    dist = "uniform" if fmt == "f32" else "normal"
    k, v, rs, rp = _seq_rows(rng, lens, Hkv, D, dist, bf16)
    q = _rows(rng, (B, Hq, D), dist, bf16)
    ks = vs = np.float32(1.0)
    if fmt == "fp8":
        ks = np.float32(np.abs(bf16_bits_to_f32(k)).max(initial=1.0) / np.float32(448.0))
        vs = np.float32(np.abs(bf16_bits_to_f32(v)).max(initial=1.0) / np.float32(448.0))
    return Workload(f"small-{fmt}-s{seed}", seed, B, Hq, Hkv, D, fmt,
                    "f32" if fmt == "f32" else "bf16", lens, nb, perm, k, v,
                    rs, rp, q, np.float32(1.0 / math.sqrt(D)), ks, vs)


@dataclasses.dataclass
class PrefixWorkload:
    """Requests that share a system prompt (retrieval-augmented generation,
    chat with a common system prompt): request r's prompt is the shared
    prefix tokens followed by its own question tokens.  KV rows of a prefix
    position are the same for every request (the KV of a position depends on
    the tokens before it, and those are shared), question rows are drawn per
    request."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    fmt: str
    prefix_ids: np.ndarray           # int32 [P]
    question_ids: List[np.ndarray]   # int32 [Q_r] per request
    prefix_k: np.ndarray             # [P, Hkv, D] source rows
    prefix_v: np.ndarray
    question_k: List[np.ndarray]     # [Q_r, Hkv, D] per request
    question_v: List[np.ndarray]
    q: np.ndarray                    # [B, Hq, D]
    num_blocks: int
    free_order: np.ndarray
    scale: np.float32

    def prompt(self, r: int) -> np.ndarray:
        return np.concatenate([self.prefix_ids, self.question_ids[r]]).astype(np.int32)

    def rows(self, r: int):
        return (np.concatenate([self.prefix_k, self.question_k[r]]),
                np.concatenate([self.prefix_v, self.question_v[r]]))


def prefix_batch(seed: int, B: int, prefix: int, qmin: int, qmax: int, Hq: int = 32,
                 Hkv: int = 8, D: int = 128, fmt: str = "bf16", vocab: int = 32000,
                 rows: bool = True) -> PrefixWorkload:
    """Draw order: prefix ids, question lengths U{qmin..qmax}, question ids,
    pool permutation, prefix K, prefix V, per request question K then V, q.
    The pool holds every request's private blocks plus the prefix once,
    times 1.25, plus 2 blocks per request of headroom."""
    rng = np.random.default_rng(seed)
    pid = rng.integers(0, vocab, prefix).astype(np.int32)
    qlen = rng.integers(qmin, qmax + 1, B)
    qid = [rng.integers(0, vocab, int(n)).astype(np.int32) for n in qlen]
    full = prefix // BLOCK
    need = full + sum(-(-(prefix + int(n)) // BLOCK) - full for n in qlen)
    nb = int(math.ceil(1.25 * need)) + 2 * B
    perm = rng.permutation(nb).astype(np.int32)
    bf16 = fmt != "f32"
    if rows:
        pk_ = _rows(rng, (prefix, Hkv, D), "normal", bf16)
        pv_ = _rows(rng, (prefix, Hkv, D), "normal", bf16)
        qk, qv = [], []
        for n in qlen:
            qk.append(_rows(rng, (int(n), Hkv, D), "normal", bf16))
            qv.append(_rows(rng, (int(n), Hkv, D), "normal", bf16))
        q = _rows(rng, (B, Hq, D), "normal", bf16)
    else:
        pk_ = pv_ = q = None
        qk = qv = []
    return PrefixWorkload(f"prefix-{fmt}-b{B}-p{prefix}", B, Hq, Hkv, D, fmt, pid, qid, pk_, pv_,
                          qk, qv, q, nb, perm, np.float32(1.0 / math.sqrt(D)))
