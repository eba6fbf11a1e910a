"""Host block manager: free pool, per-block reference counts, copy-on-write,
append-slot allocation (oracle, pure Python).

From the pages:

* The KV cache is carved into fixed 16-token blocks; each sequence has a block
  table from logical to physical block (ybb.press, "vLLM PagedAttention
  大模型推理架构深度实战", §2.2; explore.n1n.ai, "vLLM 深度解析", 映射机制详解).
* Blocks are allocated only when needed and returned as soon as a sequence
  ends; freeing is only marking, no data moves (ybb.press §2.2; unionyoga.cn,
  "vLLM：重塑大模型推理性能的关键引擎", PagedAttention section).
* The manager hands a new prompt its first blocks, and every decode iteration
  checks whether the sequence needs a new block after writing its KV
  (ybb.press, §6).
* Sequences that share a prefix share blocks, with a reference count per
  block; a sequence about to modify a block whose count exceeds one first
  copies it (ybb.press, §2.3).

Readings where the pages are silent (they make tables bit-reproducible):

* Free pool is a FIFO queue, initialised from a caller-given order (default
  0..N-1).  Allocation pops the front; a block whose count drops to zero is
  pushed to the back; a freed sequence releases its blocks in logical order.
* Appending token p (p = current length) to sequence s:
  - p % 16 == 0: pop a block, count 1, append it to s's table;
  - otherwise, if the last block's count > 1: pop b', count(b') = 1,
    count(last) -= 1, table[-1] = b', and report the copy pair (last, b');
  - slot = table[p // 16] * 16 + p % 16; length += 1.
  Full shared blocks are never copied, since appends never modify them.
* ``fork(parent, child)``: child gets a copy of the parent's table and length;
  every block in it gains one reference.
* All-or-nothing: an append that cannot get every block it needs raises
  ``NoBlocks`` and changes nothing.

Swapping (ybb.press §3.2: when device memory runs short, the KV cache of
low-priority sequences moves to CPU memory and comes back when there is room
again; §6: the scheduler swaps sequences out and in under memory pressure;
§9 item 5: swapped-out KV stays in host memory and is exchanged over the
host link).  Readings:

* A second pool of host blocks, FIFO like the device pool, initialised from
  its own order.  A sequence is either on the device or on the host; a
  swapped-out sequence cannot append, fork or be packed until swapped in.
* ``swap_out(seqs)``: every distinct device block the listed sequences
  reference, in order of first appearance (sequences in the given order,
  each table in logical order), gets one host block popped from the host
  pool; the pairs (device block, host block) are the copies to make.  Each
  table entry then points at the host copy (whose count is the number of
  entries that point at it), and the device block loses those references --
  it goes back to the device pool, in the same walk order, when its count
  reaches zero.  A block also used by sequences outside the set therefore
  stays on the device for them.
* ``swap_in(seqs)`` is the same walk from the host pool to the device pool,
  with pairs (host block, device block).
* Both are all-or-nothing: too few free blocks in the destination pool
  raise ``NoBlocks`` and change nothing; so does listing a sequence twice
  or one that is not where the call expects it (``Swapped``).
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Tuple

import numpy as np

BLOCK = 16


class NoBlocks(RuntimeError):
    pass


class UnknownSeq(KeyError):
    pass


class SeqExists(KeyError):
    pass


class Swapped(RuntimeError):
    """The sequence is not in the pool the operation needs."""


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int = BLOCK,
                 free_order: Optional[np.ndarray] = None, num_host_blocks: int = 0,
                 host_free_order: Optional[np.ndarray] = None):
        if block_size != BLOCK:
            raise ValueError("block size is 16")
        self.num_blocks = int(num_blocks)
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.free = deque(order)
        self.ref = [0] * self.num_blocks
        self.num_host_blocks = int(num_host_blocks)
        horder = (range(num_host_blocks) if host_free_order is None
                  else [int(b) for b in host_free_order])
        if sorted(horder) != list(range(num_host_blocks)):
            raise ValueError("host_free_order must be a permutation of 0..num_host_blocks-1")
        self.host_free = deque(horder)
        self.host_ref = [0] * self.num_host_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.on_host: Dict[int, bool] = {}

    # -- queries -----------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        return self.ref[block]

    def table(self, seq: int) -> List[int]:
        return list(self._get(seq))

    def length(self, seq: int) -> int:
        self._get(seq)
        return self.lens[seq]

    def num_free_host(self) -> int:
        return len(self.host_free)

    def host_refcount(self, block: int) -> int:
        return self.host_ref[block]

    def is_swapped(self, seq: int) -> bool:
        self._get(seq)
        return self.on_host[seq]

    def _get(self, seq: int) -> List[int]:
        if seq not in self.tables:
            raise UnknownSeq(seq)
        return self.tables[seq]

    def _get_dev(self, seq: int) -> List[int]:
        t = self._get(seq)
        if self.on_host[seq]:
            raise Swapped(seq)
        return t

    # -- mutations ---------------------------------------------------------
    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise SeqExists(seq)
        self.tables[seq] = []
        self.lens[seq] = 0
        self.on_host[seq] = False

    def fork(self, parent: int, child: int) -> None:
        t = self._get_dev(parent)
        if child in self.tables:
            raise SeqExists(child)
        self.tables[child] = list(t)
        self.lens[child] = self.lens[parent]
        self.on_host[child] = False
        for b in t:
            self.ref[b] += 1

    def _blocks_needed(self, seq: int, n: int) -> int:
        t = self.tables[seq]
        p = self.lens[seq]
        new = -(-(p + n) // BLOCK) - -(-p // BLOCK)
        cow = 1 if (n > 0 and p % BLOCK != 0 and self.ref[t[-1]] > 1) else 0
        return new + cow

    def append_tokens(self, seq: int, n: int) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        """Append n tokens; returns (slots, copy pair or None)."""
        self._get_dev(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        if self._blocks_needed(seq, n) > len(self.free):
            raise NoBlocks(seq)
        slots, pair = [], None
        for _ in range(n):
            s, cp = self._append_one(seq)
            slots.append(s)
            if cp is not None:
                pair = cp
        return slots, pair

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slots, pair = self.append_tokens(seq, 1)
        return slots[0], pair

    def _append_one(self, seq: int):
        t = self.tables[seq]
        p = self.lens[seq]
        pair = None
        if p % BLOCK == 0:
            b = self.free.popleft()
            self.ref[b] = 1
            t.append(b)
        elif self.ref[t[-1]] > 1:
            old = t[-1]
            b = self.free.popleft()
            self.ref[b] = 1
            self.ref[old] -= 1
            t[-1] = b
            pair = (old, b)
        slot = t[p // BLOCK] * BLOCK + p % BLOCK
        self.lens[seq] = p + 1
        return slot, pair

    def free_seq(self, seq: int) -> None:
        t = self._get(seq)
        ref, free = ((self.host_ref, self.host_free) if self.on_host[seq]
                     else (self.ref, self.free))
        for b in t:
            ref[b] -= 1
            if ref[b] == 0:
                free.append(b)
        del self.tables[seq]
        del self.lens[seq]
        del self.on_host[seq]

    # -- swapping ----------------------------------------------------------
    def _move(self, seqs, to_host: bool) -> List[Tuple[int, int]]:
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("sequence listed twice")
        for s in seqs:
            self._get(s)
            if self.on_host[s] == to_host:
                raise Swapped(s)
        src_ref, dst_ref, src_free, dst_free = (
            (self.ref, self.host_ref, self.free, self.host_free) if to_host else
            (self.host_ref, self.ref, self.host_free, self.free))
        order: List[int] = []
        for s in seqs:
            for b in self.tables[s]:
                if b not in order:
                    order.append(b)
        if len(order) > len(dst_free):
            raise NoBlocks(seqs)
        mapping = {}
        for b in order:
            mapping[b] = dst_free.popleft()
            dst_ref[mapping[b]] = 0
        for s in seqs:
            t = self.tables[s]
            for j, b in enumerate(t):
                dst_ref[mapping[b]] += 1
                src_ref[b] -= 1
                if src_ref[b] == 0:
                    src_free.append(b)
                t[j] = mapping[b]
            self.on_host[s] = to_host
        return [(b, mapping[b]) for b in order]

    def swap_out(self, seqs) -> List[Tuple[int, int]]:
        """Move the listed sequences to host blocks; (device, host) pairs."""
        return self._move(seqs, True)

    def swap_in(self, seqs) -> List[Tuple[int, int]]:
        """Move the listed sequences back to device blocks; (host, device) pairs."""
        return self._move(seqs, False)

    # -- packing -----------------------------------------------------------
    def pack(self, seq_ids, cap: int):
        """block_tables int32 [n, cap] padded with -1, context_lens int32 [n]."""
        n = len(seq_ids)
        bt = np.full((n, cap), -1, dtype=np.int32)
        cl = np.zeros(n, dtype=np.int32)
        for i, s in enumerate(seq_ids):
            t = self._get_dev(int(s))
            if len(t) > cap:
                raise ValueError("table longer than cap")
            bt[i, :len(t)] = t
            cl[i] = self.lens[int(s)]
        return bt, cl

    def check_invariants(self) -> None:
        """Counts equal table occurrences; free and referenced blocks partition
        the pool; the free queue holds no duplicates."""
        for host, n, ref, fq in ((False, self.num_blocks, self.ref, self.free),
                                 (True, self.num_host_blocks, self.host_ref, self.host_free)):
            occ = [0] * n
            for s, t in self.tables.items():
                if self.on_host[s] == host:
                    for b in t:
                        occ[b] += 1
            assert occ == ref, "refcount != table occurrences"
            free = set(fq)
            assert len(free) == len(fq), "duplicate in free queue"
            used = {b for b in range(n) if ref[b] > 0}
            assert not (free & used), "block both free and referenced"
            assert free | used == set(range(n)), "block lost"
