"""Builds the oracle's own view of a workload: block manager, caches, tables.

Everything here goes through ``oracle`` only; the GPU tests build the
library's view with the library, from the same ``workloads`` arrays.
"""
from __future__ import annotations

import numpy as np

import oracle

SENTINEL = {"f32": np.uint32(0x7FC0DEAD), "bf16": np.uint16(0x7FC1), "fp8": np.uint8(0x7F)}
STORE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def empty_cache(num_blocks, Hkv, D, fmt, bs=16):
    """A cache filled with a NaN sentinel, in storage format."""
    if fmt == "f32":
        return np.full((num_blocks, Hkv, bs, D), SENTINEL["f32"], dtype=np.uint32).view(np.float32)
    return np.full((num_blocks, Hkv, bs, D), SENTINEL[fmt], dtype=STORE[fmt])


def fill_sequential(w, cap=None):
    """Sequences 0..B-1 each get all their tokens, in sequence order, from a
    fresh manager whose free queue is ``w.free_order``; rows are written with
    ``oracle.write_kv``.  Returns (bm, k_cache, v_cache, block_tables,
    context_lens, slots_per_row)."""
    bm = oracle.RefBlockManager(w.num_blocks, free_order=w.free_order)
    per_seq = {}
    for s in range(w.B):
        bm.add_seq(s)
        per_seq[s], pair = bm.append_tokens(s, int(w.lens[s]))
        assert pair is None
    slots = np.array([per_seq[int(s)][int(p)] for s, p in zip(w.row_seq, w.row_pos)],
                     dtype=np.int64)
    kc = empty_cache(w.num_blocks, w.Hkv, w.D, w.fmt)
    vc = empty_cache(w.num_blocks, w.Hkv, w.D, w.fmt)
    kc, vc = oracle.write_kv(kc, vc, w.k_rows, w.v_rows, slots, w.src_fmt, w.fmt,
                             w.k_scale, w.v_scale)
    if cap is None:
        cap = max(1, max(-(-int(L) // 16) for L in w.lens))
    bt, cl = bm.pack(list(range(w.B)), cap)
    return bm, kc, vc, bt, cl, slots


def cow_flow_slots(bm, w):
    """The parallel-sampling flow on a block manager (oracle or library, any
    object with add_seq / append_tokens / fork): per group, the parent takes
    the prompt, three children fork from it, then every sample in ascending
    sequence id appends its suffix.  Returns (prompt slots dict, suffix slots
    dict, copy pairs in emission order)."""
    prompt_slots, suffix_slots, pairs = {}, {}, []
    for grp in w.groups:
        parent = grp["seqs"][0]
        bm.add_seq(parent)
        prompt_slots[parent], pair = bm.append_tokens(parent, grp["prompt"])
        assert pair is None
    for grp in w.groups:
        for child in grp["seqs"][1:]:
            bm.fork(grp["seqs"][0], child)
    for grp in w.groups:
        for sid, sl in zip(grp["seqs"], grp["suffix"]):
            suffix_slots[sid], pair = bm.append_tokens(sid, sl)
            if pair is not None:
                pairs.append(pair)
    return prompt_slots, suffix_slots, pairs


def row_slots_cow(w, prompt_slots, suffix_slots):
    """Slot of every row of the copy-on-write workload (prompt rows map to the
    parent's slots, suffix rows to the sample's)."""
    out = np.empty(len(w.row_seq), dtype=np.int64)
    first = {g["seqs"][0]: g for g in w.groups}
    for i, (s, p) in enumerate(zip(w.row_seq, w.row_pos)):
        s, p = int(s), int(p)
        if s in first and p < first[s]["prompt"]:
            out[i] = prompt_slots[s][p]
        else:
            grp = w.groups[s // 4]
            out[i] = suffix_slots[s][p - grp["prompt"]]
    return out


def is_prompt_row(w):
    first = {g["seqs"][0]: g["prompt"] for g in w.groups}
    return np.array([int(s) in first and int(p) < first[int(s)]
                     for s, p in zip(w.row_seq, w.row_pos)])


def fill_cow(w):
    """Oracle view of the parallel-sampling workload: prompt written, forks,
    suffix appends, block copies, suffix written."""
    bm = oracle.RefBlockManager(w.num_blocks, free_order=w.free_order)
    ps, ss, pairs = cow_flow_slots(bm, w)
    slots = row_slots_cow(w, ps, ss)
    prompt = is_prompt_row(w)
    kc = empty_cache(w.num_blocks, w.Hkv, w.D, w.fmt)
    vc = empty_cache(w.num_blocks, w.Hkv, w.D, w.fmt)
    kc, vc = oracle.write_kv(kc, vc, w.k_rows[prompt], w.v_rows[prompt], slots[prompt],
                             w.src_fmt, w.fmt, w.k_scale, w.v_scale)
    kc, vc = oracle.copy_blocks(kc, vc, pairs)
    kc, vc = oracle.write_kv(kc, vc, w.k_rows[~prompt], w.v_rows[~prompt], slots[~prompt],
                             w.src_fmt, w.fmt, w.k_scale, w.v_scale)
    cap = max(-(-int(L) // 16) for L in w.lens)
    bt, cl = bm.pack(list(range(w.B)), cap)
    return bm, kc, vc, bt, cl, pairs


def contiguous_rows(w, s):
    """Rows of sequence s in position order, straight from the generator."""
    idx = np.nonzero(w.row_seq == s)[0]
    order = np.argsort(w.row_pos[idx], kind="stable")
    return w.k_rows[idx[order]], w.v_rows[idx[order]]
