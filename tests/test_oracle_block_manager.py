"""Pins of the oracle block manager: hand-worked traces of the rules,
closed forms on fresh pools, invariants under random operation scripts."""
import numpy as np
import pytest

import oracle
import workloads
from tests._oracle_setup import cow_flow_slots


def test_hand_worked_fork_and_copy_on_write_trace():
    """Pool of 6 blocks, free order [5, 3, 0, 1, 4, 2]; derived by hand from
    the append / fork / copy-on-write / free rules."""
    bm = oracle.RefBlockManager(6, free_order=[5, 3, 0, 1, 4, 2])
    bm.add_seq(10)
    slots, pair = bm.append_tokens(10, 18)     # blocks 5 (full), 3 (2 slots)
    assert pair is None
    assert slots[:16] == list(range(80, 96)) and slots[16:] == [48, 49]
    bm.fork(10, 11)
    bm.fork(10, 12)
    assert bm.refcount(5) == 3 and bm.refcount(3) == 3
    # 10 appends into the shared partial block 3 -> copies it to block 0
    s, pair = bm.append_slot(10)
    assert pair == (3, 0) and s == 0 * 16 + 2
    # 12 appends: block 3 still shared by 11 and 12 -> copy to block 1
    s, pair = bm.append_slot(12)
    assert pair == (3, 1) and s == 16 + 2
    # 11 is now the only owner of block 3: writes in place
    s, pair = bm.append_slot(11)
    assert pair is None and s == 3 * 16 + 2
    assert bm.table(10) == [5, 0] and bm.table(11) == [5, 3] and bm.table(12) == [5, 1]
    assert bm.refcount(5) == 3 and [bm.refcount(b) for b in (0, 1, 3)] == [1, 1, 1]
    # full shared block 5 is never copied: 10 fills block 0, then gets block 4
    slots, pair = bm.append_tokens(10, 14)
    assert pair is None and slots[-1] == 4 * 16 + 0
    assert bm.table(10) == [5, 0, 4]
    bm.free_seq(10)                             # releases 0 and 4 (5 still shared)
    assert list(bm.free) == [2, 0, 4]
    bm.free_seq(11)
    bm.free_seq(12)                             # 5 freed here, then 1
    assert list(bm.free) == [2, 0, 4, 3, 5, 1]
    assert bm.num_free() == 6


def test_fresh_pool_tables_are_consecutive_free_order_entries():
    w = workloads.config3(rows=False)
    bm = oracle.RefBlockManager(w.num_blocks, free_order=w.free_order)
    pos = 0
    for s in range(w.B):
        bm.add_seq(s)
        slots, _ = bm.append_tokens(s, int(w.lens[s]))
        n = -(-int(w.lens[s]) // 16)
        assert bm.table(s) == list(w.free_order[pos:pos + n])
        t = np.arange(int(w.lens[s]))
        exp = w.free_order[pos + t // 16].astype(np.int64) * 16 + t % 16
        assert slots == list(exp)
        pos += n
    assert pos == 11583
    bm.check_invariants()


def test_parallel_sampling_workload_gives_192_copies():
    w = workloads.config5(rows=False)
    bm = oracle.RefBlockManager(w.num_blocks, free_order=w.free_order)
    ps, ss, pairs = cow_flow_slots(bm, w)
    assert len(pairs) == 192
    bm.check_invariants()
    for grp in w.groups:
        parent = grp["seqs"][0]
        t = bm.table(parent)
        # the 64 full prompt blocks are still shared by all four samples
        for b in t[:64]:
            assert bm.refcount(b) == 4
        for sid in grp["seqs"]:
            assert bm.table(sid)[:64] == t[:64]
    # three copies per group, made by the first three samples in id order
    per_group = {}
    for (src, dst) in pairs:
        per_group.setdefault(src, []).append(dst)
    assert all(len(v) == 3 for v in per_group.values()) and len(per_group) == 64


def test_block_aligned_prompt_needs_no_copy():
    w = workloads.config5(rows=False, aligned=True)
    bm = oracle.RefBlockManager(w.num_blocks, free_order=w.free_order)
    _, _, pairs = cow_flow_slots(bm, w)
    assert pairs == []


def test_out_of_blocks_changes_nothing():
    bm = oracle.RefBlockManager(3)
    bm.add_seq(0)
    bm.append_tokens(0, 17)
    bm.fork(0, 1)
    before = (list(bm.free), list(bm.ref), bm.table(0), bm.length(0))
    with pytest.raises(oracle.NoBlocks):
        bm.append_tokens(0, 32)          # needs a copy + 2 new blocks, 1 free
    assert (list(bm.free), list(bm.ref), bm.table(0), bm.length(0)) == before
    bm.append_tokens(0, 15)              # copy only: fits
    with pytest.raises(oracle.NoBlocks):
        bm.append_slot(0)
    with pytest.raises(oracle.UnknownSeq):
        bm.append_slot(7)
    with pytest.raises(oracle.SeqExists):
        bm.fork(0, 1)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_invariants_hold_under_random_scripts(seed):
    rng = np.random.default_rng(seed)
    bm = oracle.RefBlockManager(64, free_order=rng.permutation(64))
    live, next_id = [], 0
    for _ in range(3000):
        op = rng.integers(0, 10)
        try:
            if op == 0 or not live:
                bm.add_seq(next_id)
                live.append(next_id)
                next_id += 1
            elif op == 1:
                bm.fork(int(rng.choice(live)), next_id)
                live.append(next_id)
                next_id += 1
            elif op == 2:
                s = int(rng.choice(live))
                bm.free_seq(s)
                live.remove(s)
            else:
                s = int(rng.choice(live))
                n = int(rng.integers(1, 20))
                L0, t0 = bm.length(s), bm.table(s)
                slots, pair = bm.append_tokens(s, n)
                t = bm.table(s)
                # slots are the consecutive positions of the sequence
                assert slots == [t[p // 16] * 16 + p % 16 for p in range(L0, L0 + n)]
                # a copy replaces exactly the old last block
                if pair is not None:
                    assert L0 % 16 != 0 and pair[0] == t0[-1] and t[len(t0) - 1] == pair[1]
        except oracle.NoBlocks:
            pass
        bm.check_invariants()
    for s in list(live):
        bm.free_seq(s)
    assert bm.num_free() == 64
