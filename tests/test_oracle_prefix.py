"""Pins of the oracle's prefix caching: the FNV-1a hash against its
published test vectors, hand-worked traces of reuse and eviction, the hit
rate of a shared-prompt workload in closed form, no sharing under forced
hash collisions, and invariants under random scripts."""
import numpy as np
import pytest

import oracle
import oracle.block_manager as obm


def test_fnv1a64_published_vectors():
    assert obm.fnv1a64(b"") == 0xCBF29CE484222325
    assert obm.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert obm.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_key_chains_parent_and_tokens():
    toks = list(range(16))
    k0 = oracle.block_key(0, toks)
    assert k0 == obm.fnv1a64(bytes(8) + b"".join(t.to_bytes(4, "little") for t in toks))
    assert oracle.block_key(k0, toks) != k0                      # the parent matters
    assert oracle.block_key(0, toks[::-1]) != k0                  # the order matters
    assert oracle.block_key(0, [-1] + toks[1:]) == obm.fnv1a64(
        bytes(8) + (-1).to_bytes(4, "little", signed=True) + b"".join(
            t.to_bytes(4, "little") for t in toks[1:]))


def _mgr(n=16):
    bm = oracle.RefBlockManager(n)
    bm.enable_prefix_caching()
    return bm


def test_hand_worked_reuse_and_eviction_trace():
    bm = _mgr(6)
    a = list(range(100, 140))                 # 2 full blocks + 8
    b = a[:32] + [7, 8, 9, 10, 11]            # same 2 full blocks, other tail
    slots, nc = bm.add_seq_prompt(0, a)
    assert nc == 0 and bm.table(0) == [0, 1, 2]
    assert bm.cache_stats() == (2, 0, 2, 0)   # blocks 0 and 1 registered
    slots, nc = bm.add_seq_prompt(1, b)
    assert nc == 32 and bm.table(1) == [0, 1, 3]
    assert slots[:32] == list(range(32)) and slots[32] == 3 * 16
    assert [bm.refcount(x) for x in range(4)] == [2, 2, 1, 1]
    assert bm.cache_stats() == (4, 2, 2, 0)
    bm.free_seq(0)
    bm.free_seq(1)                            # 0, 1 evictable (in that order); 2, 3 free
    assert list(bm.free) == [4, 5, 2, 3] and list(bm.lru) == [0, 1]
    assert bm.num_free() == 6
    # a prompt sharing only the first block revives block 0
    c = a[:16] + [1] * 16
    slots, nc = bm.add_seq_prompt(2, c)
    assert nc == 16 and bm.table(2) == [0, 4] and list(bm.lru) == [1]
    # its second block is full and new: registered
    assert bm.cache_stats()[2] == 3
    # take every remaining block: free ones first, then block 1 is evicted
    bm.add_seq(3)
    bm.append_tokens(3, 16 * 4)               # 5, 2, 3, then evicts 1
    assert bm.table(3) == [5, 2, 3, 1] and not bm.lru and 1 not in bm.bkey
    bm.free_seq(3)
    # a's second block is gone from the cache: only one block hits now
    slots, nc = bm.add_seq_prompt(4, a)
    assert nc == 16 and bm.table(4)[0] == 0
    bm.check_invariants()


def test_rag_workload_hit_rate_closed_form():
    """R requests share a P-token system prompt (P a multiple of 16) and add
    their own question; served one at a time.  The first misses everything;
    every later one hits the P/16 prompt blocks."""
    rng = np.random.default_rng(0)
    R, P = 20, 512
    system = list(rng.integers(0, 32000, P))
    bm = _mgr(400)
    queried = hits = 0
    for r in range(R):
        q = list(rng.integers(0, 32000, int(rng.integers(10, 200))))
        toks = system + q
        slots, nc = bm.add_seq_prompt(r, toks)
        assert nc == (0 if r == 0 else P)
        queried += len(toks) // 16
        hits += 0 if r == 0 else P // 16
        bm.append_token_ids(r, list(rng.integers(0, 32000, 30)))   # generated answer
        bm.free_seq(r)
    assert bm.cache_stats()[:2] == (queried, hits)
    assert hits / queried > 0.7
    bm.check_invariants()


def test_forced_collisions_never_share_blocks(monkeypatch):
    """With every key colliding, only exact (parent, tokens) matches may be
    reused: different prompts get their own blocks."""
    monkeypatch.setattr(obm, "block_key", lambda parent, toks: 42)
    bm = _mgr(10)
    bm.add_seq_prompt(0, list(range(32)))
    slots, nc = bm.add_seq_prompt(1, list(range(1, 33)))
    assert nc == 0 and set(bm.table(1)).isdisjoint(bm.table(0))
    slots, nc = bm.add_seq_prompt(2, list(range(16)) + [5] * 16)
    assert nc == 16 and bm.table(2)[0] == bm.table(0)[0]


def test_capacity_check_counts_revived_blocks():
    bm = _mgr(3)
    bm.add_seq_prompt(0, list(range(32)))     # blocks 0, 1 registered
    bm.free_seq(0)                            # both evictable, 1 free block
    assert bm.num_free() == 3
    # reusing both blocks leaves one block for a 3rd: fits exactly
    slots, nc = bm.add_seq_prompt(1, list(range(32)) + [9] * 16)
    assert nc == 32 and bm.num_free() == 0
    bm.free_seq(1)
    # a prompt hitting block 0 only needs 2 more, and 2 remain besides it
    with pytest.raises(oracle.NoBlocks):
        bm.add_seq_prompt(2, list(range(16)) + [3] * 48)
    bm.check_invariants()


def test_appending_without_ids_stops_registration():
    bm = _mgr(8)
    bm.add_seq_prompt(0, list(range(20)))
    bm.append_tokens(0, 12)                   # ids unknown: block 1 fills unregistered
    assert bm.cache_stats()[2] == 1
    slots, nc = bm.add_seq_prompt(1, list(range(32)))
    assert nc == 16


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_invariants_hold_under_random_prompt_scripts(seed):
    rng = np.random.default_rng(seed)
    bm = oracle.RefBlockManager(60, free_order=rng.permutation(60), num_host_blocks=30)
    bm.enable_prefix_caching()
    prefixes = [list(rng.integers(0, 50, int(rng.integers(0, 80)))) for _ in range(4)]
    live, nxt = [], 0
    for _ in range(2500):
        op = int(rng.integers(0, 10))
        dev = [s for s in live if not bm.is_swapped(s)]
        try:
            if op <= 2 or not live:
                toks = prefixes[int(rng.integers(0, 4))] + list(rng.integers(0, 50, int(rng.integers(0, 40))))
                q0, h0, _, _ = bm.cache_stats()
                slots, nc = bm.add_seq_prompt(nxt, toks)
                t = bm.table(nxt)
                assert nc % 16 == 0 and nc <= len(toks) and len(slots) == len(toks)
                assert slots == [t[p // 16] * 16 + p % 16 for p in range(len(toks))]
                live.append(nxt)
                nxt += 1
            elif op == 3:
                s = live[int(rng.integers(len(live)))]
                bm.free_seq(s)
                live.remove(s)
            elif op == 4 and dev:
                bm.fork(dev[int(rng.integers(len(dev)))], nxt)
                live.append(nxt)
                nxt += 1
            elif op == 5 and dev:
                bm.swap_out([dev[int(rng.integers(len(dev)))]])
            elif op == 6 and len(dev) < len(live):
                host = [s for s in live if bm.is_swapped(s)]
                bm.swap_in([host[int(rng.integers(len(host)))]])
            elif dev:
                s = dev[int(rng.integers(len(dev)))]
                bm.append_token_ids(s, list(rng.integers(0, 50, int(rng.integers(1, 20)))))
        except oracle.NoBlocks:
            pass
        bm.check_invariants()


def test_shared_prefix_groups_hand_worked():
    """Requests 0..2 share a 40-token prompt (2 full blocks), request 3 has
    its own prompt, requests 4..5 share a 20-token prompt (1 full block),
    request 6 repeats the first prompt after them: runs are of adjacent
    sequences only, and a shared block must leave each member a token."""
    bm = oracle.RefBlockManager(64)
    bm.enable_prefix_caching()
    a = list(range(100, 140))
    b = list(range(200, 220))
    prompts = [a + [1, 2], a + [3], a + [4, 5, 6, 7], [9] * 30, b + [1], b + [2, 3], a + [8]]
    for s, p in enumerate(prompts):
        bm.add_seq_prompt(s, p)
    assert bm.shared_prefix_groups(range(7)) == [(0, 3, 2), (4, 2, 1)]
    # the same sequences in another order: runs follow the order given
    assert bm.shared_prefix_groups([6, 0, 3, 1, 2]) == [(0, 2, 2), (3, 2, 2)]
    # a member whose whole length is the shared blocks caps the run one block
    # lower (32 tokens: blocks 0, 1 full, nothing after them)
    bm.add_seq_prompt(7, a[:32])
    assert bm.table(7) == bm.table(0)[:2]
    assert bm.shared_prefix_groups([0, 7, 1]) == [(0, 3, 1)]
    # forks share every block, the partial last one included, but the
    # shared run stops at the full blocks below each length
    bm.fork(3, 8)
    assert bm.shared_prefix_groups([3, 8]) == [(0, 2, 1)]
    assert bm.shared_prefix_groups([3]) == [] and bm.shared_prefix_groups([]) == []


def _groups_brute(bm, ids):
    """Every split of ids into runs, scored: a run of two or more whose members
    agree on their first k table entries and have more than k*bs tokens, for
    the largest such k >= 1."""
    out, i = [], 0
    tabs = [bm.table(s) for s in ids]
    lens = [bm.length(s) for s in ids]
    while i < len(ids):
        j = i + 1
        while j < len(ids) and tabs[j][:1] and tabs[j][:1] == tabs[i][:1]:
            j += 1
        best = 0
        for k in range(1, 1 + max(len(t) for t in tabs[i:j])):
            if all(len(tabs[r]) >= k and tabs[r][:k] == tabs[i][:k] and lens[r] > k * bm.bs
                   for r in range(i, j)):
                best = k
        if j - i >= 2 and best >= 1:
            out.append((i, j - i, best))
        i = j
    return out


@pytest.mark.parametrize("seed,bs", [(11, 16), (12, 8), (13, 32)])
def test_shared_prefix_groups_against_brute_force(seed, bs):
    rng = np.random.default_rng(seed)
    bm = oracle.RefBlockManager(400, block_size=bs)
    bm.enable_prefix_caching()
    prompts = [[int(x) for x in rng.integers(0, 50, int(rng.integers(0, 100)))] for _ in range(4)]
    live = []
    for s in range(60):
        if live and rng.random() < 0.2:
            bm.fork(int(rng.choice(live)), s)
        else:
            bm.add_seq_prompt(s, prompts[int(rng.integers(0, 4))] +
                              [int(x) for x in rng.integers(0, 50, int(rng.integers(0, 20)))])
        live.append(s)
    for _ in range(20):
        ids = sorted(live, key=lambda s: (bm.table(s)[:1], rng.random()))
        assert bm.shared_prefix_groups(ids) == _groups_brute(bm, ids)
