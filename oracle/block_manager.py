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

* Block size: 16 tokens, as the pages state is usual; 8, 32 and 64 are also
  accepted, since the block size is to be tuned to typical request lengths
  (unionyoga.cn, section "在真实架构中扮演什么角色？").  Every rule below uses
  the manager's block size where it says 16.

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

Prefix caching (explore.n1n.ai, "vLLM 深度解析", section "vLLM 生态的核心功能
亮点": requests that share a system prompt or documents reuse that prefix's
cached KV instead of recomputing it; ybb.press §7.3: automatic prefix caching
finds identical prefixes across requests and shares their KV blocks, e.g.
earlier turns of a chat; gheillcoat.github.io, "概念-vLLM", section 3: shared
prefixes such as the system prompt are cached automatically; unionyoga.cn,
section "在真实架构中扮演什么角色？": block-cache hit rate is a monitored
figure, target above 95%).  Readings:

* Once enabled, a full block written through the token-id calls gets a key:
  FNV-1a 64 (the published Fowler-Noll-Vo hash) over the 8 little-endian
  bytes of its parent's key (0 for a sequence's first block) followed by its
  16 token ids as 4-byte little-endian integers.  The first block with a key
  is registered for it; the key chain makes the key depend on the whole
  prefix.
* ``add_seq_prompt(seq, tokens)``: the longest run of the prompt's leading
  full blocks whose keys are registered -- and whose stored parent key and
  tokens match, so a hash collision is never shared -- is reused (each
  block gains a reference); the caller need not write those tokens' KV
  (``num_cached``).  The rest of the prompt is appended.  Queried blocks =
  the prompt's full blocks; hit blocks = the reused ones.
* A registered block whose count drops to zero is not freed but becomes
  evictable, most recently released last; a hit revives it.  Allocation
  takes the free queue first, then evicts the least recently released
  block (dropping its registration).  Capacity checks count both.
* Appending without token ids stops a sequence's blocks being registered.
"""
from __future__ import annotations

from collections import OrderedDict, deque
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16
BLOCK_SIZES = (8, 16, 32, 64)

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit: for each byte, h ^= byte, then h *= prime (mod 2^64)."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_key(parent: int, tokens: Sequence[int]) -> int:
    """FNV-1a 64 over parent key (8 bytes LE) then the token ids (4 bytes LE each)."""
    return fnv1a64(int(parent).to_bytes(8, "little") + b"".join(
        int(t).to_bytes(4, "little", signed=True) for t in tokens))


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
        if block_size not in BLOCK_SIZES:
            raise ValueError(f"block size must be one of {BLOCK_SIZES}")
        self.bs = int(block_size)
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
        # prefix caching
        self.caching = False
        self.cache: Dict[int, int] = {}                 # key -> block
        self.bkey: Dict[int, int] = {}                  # registered block -> key
        self.bmeta: Dict[int, Tuple[int, tuple]] = {}   # registered block -> (parent key, tokens)
        self.lru: "OrderedDict[int, None]" = OrderedDict()   # evictable, oldest release first
        self.toks: Dict[int, Optional[List[int]]] = {}  # token ids (None: not tracked)
        self.last_key: Dict[int, int] = {}
        self.queried = 0
        self.hits = 0

    def enable_prefix_caching(self) -> None:
        self.caching = True

    def available(self) -> int:
        return len(self.free) + len(self.lru)

    def cache_stats(self):
        """(queried blocks, hit blocks, registered blocks, evictable blocks)."""
        return self.queried, self.hits, len(self.cache), len(self.lru)

    def _pop(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:
            b, _ = self.lru.popitem(last=False)
            del self.cache[self.bkey.pop(b)]
            del self.bmeta[b]
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        """A device block's count reached zero."""
        if b in self.bkey:
            self.lru[b] = None
        else:
            self.free.append(b)

    # -- queries -----------------------------------------------------------
    def num_free(self) -> int:
        """Blocks an allocation can take: free plus evictable."""
        return self.available()

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
        self.toks[seq] = [] if self.caching else None
        self.last_key[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        t = self._get_dev(parent)
        if child in self.tables:
            raise SeqExists(child)
        self.tables[child] = list(t)
        self.lens[child] = self.lens[parent]
        self.on_host[child] = False
        self.toks[child] = None if self.toks[parent] is None else list(self.toks[parent])
        self.last_key[child] = self.last_key[parent]
        for b in t:
            self.ref[b] += 1

    def _blocks_needed(self, seq: int, n: int) -> int:
        t = self.tables[seq]
        p = self.lens[seq]
        new = -(-(p + n) // self.bs) - -(-p // self.bs)
        cow = 1 if (n > 0 and p % self.bs != 0 and self.ref[t[-1]] > 1) else 0
        return new + cow

    def append_tokens(self, seq: int, n: int) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        """Append n tokens; returns (slots, copy pair or None).  Their ids are
        unknown, so the sequence's blocks stop being registered."""
        return self._append(seq, n, None)

    def append_token_ids(self, seq: int, tokens) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        """Append tokens with their ids (full blocks get registered)."""
        return self._append(seq, len(tokens), [int(t) for t in tokens])

    def _append(self, seq, n, ids):
        self._get_dev(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        if self._blocks_needed(seq, n) > self.available():
            raise NoBlocks(seq)
        if ids is None and n > 0:
            self.toks[seq] = None
        slots, pair = [], None
        for i in range(n):
            s, cp = self._append_one(seq)
            slots.append(s)
            if cp is not None:
                pair = cp
            if ids is not None:
                self._note_token(seq, ids[i])
        return slots, pair

    def _note_token(self, seq: int, tok: int) -> None:
        tk = self.toks[seq]
        if tk is None:
            return
        tk.append(tok)
        if len(tk) % self.bs == 0:                     # a block just filled
            blk = tuple(tk[-self.bs:])
            key = block_key(self.last_key[seq], blk)
            b = self.tables[seq][len(tk) // self.bs - 1]
            if key not in self.cache and b not in self.bkey:
                self.cache[key] = b
                self.bkey[b] = key
                self.bmeta[b] = (self.last_key[seq], blk)
            self.last_key[seq] = key

    def add_seq_prompt(self, seq: int, tokens) -> Tuple[List[int], int]:
        """New sequence with a prompt: reuse the longest cached run of its
        leading full blocks, append the rest.  Returns (slots, num_cached)."""
        if seq in self.tables:
            raise SeqExists(seq)
        tokens = [int(t) for t in tokens]
        hits: List[int] = []
        parent = 0
        if self.caching:
            for k in range(len(tokens) // self.bs):
                blk = tuple(tokens[self.bs * k:self.bs * (k + 1)])
                key = block_key(parent, blk)
                b = self.cache.get(key)
                if b is None or self.bmeta[b] != (parent, blk):
                    break
                hits.append(b)
                parent = key
        revived = sum(1 for b in hits if self.ref[b] == 0)
        need = -(-len(tokens) // self.bs) - len(hits)
        if need > self.available() - revived:
            raise NoBlocks(seq)
        self.add_seq(seq)
        if self.caching:
            self.queried += len(tokens) // self.bs
            self.hits += len(hits)
        t = self.tables[seq]
        for b in hits:
            if self.ref[b] == 0:
                del self.lru[b]
            self.ref[b] += 1
            t.append(b)
        nc = self.bs * len(hits)
        self.lens[seq] = nc
        if self.toks[seq] is not None:
            self.toks[seq] = tokens[:nc]
        self.last_key[seq] = parent
        slots = [t[p // self.bs] * self.bs + p % self.bs for p in range(nc)]
        more, pair = self.append_token_ids(seq, tokens[nc:])
        assert pair is None
        return slots + more, nc

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slots, pair = self.append_tokens(seq, 1)
        return slots[0], pair

    def _append_one(self, seq: int):
        t = self.tables[seq]
        p = self.lens[seq]
        pair = None
        if p % self.bs == 0:
            b = self._pop()
            t.append(b)
        elif self.ref[t[-1]] > 1:
            old = t[-1]
            b = self._pop()
            self.ref[old] -= 1
            t[-1] = b
            pair = (old, b)
        slot = t[p // self.bs] * self.bs + p % self.bs
        self.lens[seq] = p + 1
        return slot, pair

    def free_seq(self, seq: int) -> None:
        t = self._get(seq)
        for b in t:
            if self.on_host[seq]:
                self.host_ref[b] -= 1
                if self.host_ref[b] == 0:
                    self.host_free.append(b)
            else:
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self._release(b)
        del self.tables[seq]
        del self.lens[seq]
        del self.on_host[seq]
        del self.toks[seq]
        del self.last_key[seq]

    # -- swapping ----------------------------------------------------------
    def _move(self, seqs, to_host: bool) -> List[Tuple[int, int]]:
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("sequence listed twice")
        for s in seqs:
            self._get(s)
            if self.on_host[s] == to_host:
                raise Swapped(s)
        src_ref, dst_ref = (self.ref, self.host_ref) if to_host else (self.host_ref, self.ref)
        order: List[int] = []
        for s in seqs:
            for b in self.tables[s]:
                if b not in order:
                    order.append(b)
        room = len(self.host_free) if to_host else self.available()
        if len(order) > room:
            raise NoBlocks(seqs)
        mapping = {}
        for b in order:
            if to_host:
                mapping[b] = self.host_free.popleft()
            else:
                mapping[b] = self._pop()
            dst_ref[mapping[b]] = 0
        for s in seqs:
            t = self.tables[s]
            for j, b in enumerate(t):
                dst_ref[mapping[b]] += 1
                src_ref[b] -= 1
                if src_ref[b] == 0:
                    if to_host:
                        self._release(b)
                    else:
                        self.host_free.append(b)
                t[j] = mapping[b]
            self.on_host[s] = to_host
        return [(b, mapping[b]) for b in order]

    def swap_out(self, seqs) -> List[Tuple[int, int]]:
        """Move the listed sequences to host blocks; (device, host) pairs."""
        return self._move(seqs, True)

    def swap_in(self, seqs) -> List[Tuple[int, int]]:
        """Move the listed sequences back to device blocks; (host, device) pairs."""
        return self._move(seqs, False)

    # -- shared prefixes ---------------------------------------------------
    def shared_prefix_groups(self, seq_ids) -> List[Tuple[int, int, int]]:
        """Runs of adjacent sequences (in the given order) whose tables start
        with the same block, as (index of the first, count, shared blocks):
        shared = the longest common run of leading table entries that are
        full blocks and leave every member at least one more token
        (shared * bs < L).  Runs of one sequence, or with no shared block,
        are left out.  Reading: the pages say requests with a common prefix
        share its blocks; attention over such a prefix is computed once for
        all of them."""
        ids = [int(s) for s in seq_ids]
        out = []
        i = 0
        while i < len(ids):
            t0 = self._get_dev(ids[i])
            j = i + 1
            while j < len(ids) and self._get_dev(ids[j])[:1] == t0[:1] and t0:
                j += 1
            if j - i >= 2:
                m = min((self.lens[ids[k]] - 1) // self.bs for k in range(i, j))
                for k in range(i + 1, j):
                    t = self.tables[ids[k]]
                    c = 0
                    while c < min(len(t), len(t0)) and t[c] == t0[c]:
                        c += 1
                    m = min(m, c)
                if m >= 1:
                    out.append((i, j - i, m))
            i = j
        return out

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
            free = set(fq) | (set() if host else set(self.lru))
            assert len(free) == len(fq) + (0 if host else len(self.lru)), "duplicate in free pools"
            used = {b for b in range(n) if ref[b] > 0}
            assert not (free & used), "block both free and referenced"
            assert free | used == set(range(n)), "block lost"
        assert set(self.lru) <= set(self.bkey), "evictable block not registered"
        assert all(self.cache[k] == b for b, k in self.bkey.items()), "registry out of sync"
        assert len(self.cache) == len(self.bkey)
