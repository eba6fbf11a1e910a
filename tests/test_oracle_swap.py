"""Pins of the oracle's swapping (host block pool, swap_out / swap_in,
swap_blocks) to hand-worked traces, invariants and a data round trip that
decode checks."""
import numpy as np
import pytest

import oracle
import workloads
from tests._oracle_setup import fill_sequential


def _state(bm):
    return (dict((s, list(t)) for s, t in bm.tables.items()), list(bm.ref), list(bm.host_ref),
            list(bm.free), list(bm.host_free), dict(bm.on_host), dict(bm.lens))


def test_hand_worked_swap_trace():
    bm = oracle.RefBlockManager(8, num_host_blocks=6)
    bm.add_seq(0)
    bm.append_tokens(0, 20)                 # blocks 0, 1
    bm.fork(0, 1)                           # 1 shares 0, 1
    bm.add_seq(2)
    bm.append_tokens(2, 5)                  # block 2
    assert list(bm.free) == [3, 4, 5, 6, 7]
    # sequence 1 alone: both its blocks get host copies 0, 1; they stay on
    # the device for sequence 0
    assert bm.swap_out([1]) == [(0, 0), (1, 1)]
    assert bm.table(1) == [0, 1] and bm.is_swapped(1)
    assert bm.ref[:3] == [1, 1, 1] and bm.host_ref[:2] == [1, 1]
    assert list(bm.free) == [3, 4, 5, 6, 7] and list(bm.host_free) == [2, 3, 4, 5]
    # sequences 0 and 2: three more host blocks; the device blocks free up
    # in walk order
    assert bm.swap_out([0, 2]) == [(0, 2), (1, 3), (2, 4)]
    assert bm.table(0) == [2, 3] and bm.table(2) == [4]
    assert list(bm.free) == [3, 4, 5, 6, 7, 0, 1, 2] and list(bm.host_free) == [5]
    assert bm.ref == [0] * 8
    # back in: sequence 1 takes device blocks 3, 4; its host blocks free up
    assert bm.swap_in([1]) == [(0, 3), (1, 4)]
    assert bm.table(1) == [3, 4] and not bm.is_swapped(1)
    assert list(bm.host_free) == [5, 0, 1]
    # a swapped-in sequence appends again (token 20 goes to block 4, offset 4)
    assert bm.append_slot(1) == (4 * 16 + 4, None)
    bm.check_invariants()


def test_sharers_swapped_together_keep_sharing():
    bm = oracle.RefBlockManager(10, num_host_blocks=10)
    bm.add_seq(0)
    bm.append_tokens(0, 40)                 # 0, 1, 2
    for c in (1, 2, 3):
        bm.fork(0, c)
    pairs = bm.swap_out([0, 1, 2, 3])
    assert pairs == [(0, 0), (1, 1), (2, 2)]                  # each block copied once
    assert bm.host_ref[:3] == [4, 4, 4] and all(bm.table(s) == [0, 1, 2] for s in range(4))
    assert bm.num_free() == 10
    pairs = bm.swap_in([2, 0, 3, 1])
    assert len(pairs) == 3 and all(bm.table(s) == bm.table(2) for s in range(4))
    # a partial shared last block still gets copied on write after the round trip
    slot, pair = bm.append_slot(3)
    assert pair is not None and pair[0] == bm.table(0)[2]
    bm.check_invariants()


def test_swap_is_all_or_nothing_and_guards_swapped_sequences():
    bm = oracle.RefBlockManager(8, num_host_blocks=2)
    bm.add_seq(0)
    bm.append_tokens(0, 40)                 # 3 blocks
    bm.add_seq(1)
    bm.append_tokens(1, 3)
    before = _state(bm)
    with pytest.raises(oracle.NoBlocks):
        bm.swap_out([0])                    # needs 3 host blocks, 2 free
    assert _state(bm) == before
    with pytest.raises(ValueError):
        bm.swap_out([1, 1])
    assert _state(bm) == before
    assert bm.swap_out([1]) == [(3, 0)]
    for call in (lambda: bm.append_slot(1), lambda: bm.fork(1, 5),
                 lambda: bm.pack([0, 1], 4), lambda: bm.swap_out([1]),
                 lambda: bm.swap_in([0])):
        snap = _state(bm)
        with pytest.raises(oracle.Swapped):
            call()
        assert _state(bm) == snap
    bm.free_seq(1)                          # freeing a swapped sequence frees host blocks
    assert bm.num_free_host() == 2
    bm.check_invariants()


def test_swap_round_trip_through_host_pool_preserves_decode_bitwise():
    """Swap a subset out (copying the blocks to a host pool), let other
    sequences reuse the freed device blocks, swap back in to different
    blocks: decode of every sequence is bit-identical to before."""
    w = workloads.small_random(91, 6, 8, 2, 16, "bf16", 90, 20)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    bm2 = oracle.RefBlockManager(w.num_blocks + 40, free_order=np.r_[w.free_order,
                                 np.arange(w.num_blocks, w.num_blocks + 40)],
                                 num_host_blocks=40, host_free_order=np.arange(40)[::-1])
    for s in range(w.B):
        bm2.add_seq(s)
        bm2.append_tokens(s, int(w.lens[s]))
    shape = (w.num_blocks + 40, w.Hkv, 16, w.D)
    kc2 = np.zeros(shape, np.uint16)
    vc2 = np.zeros(shape, np.uint16)
    kc2[:w.num_blocks], vc2[:w.num_blocks] = kc, vc
    bt0, cl0 = bm2.pack(range(w.B), 8)
    ref = oracle.decode(w.q, "bf16", kc2, vc2, "bf16", bt0, cl0, w.scale)
    hk = np.zeros((40, w.Hkv, 16, w.D), np.uint16)
    hv = np.zeros_like(hk)
    out_pairs = bm2.swap_out([4, 1])
    hk, hv = oracle.swap_blocks(kc2, vc2, hk, hv, out_pairs)
    # the freed device blocks are reused and overwritten by another sequence
    bm2.add_seq(99)
    slots, _ = bm2.append_tokens(99, 16 * bm2.num_free())
    kc2[np.asarray(slots) // 16, :, np.asarray(slots) % 16] = 0x7FC1
    vc2[np.asarray(slots) // 16, :, np.asarray(slots) % 16] = 0x7FC1
    bm2.free_seq(99)
    in_pairs = bm2.swap_in([1, 4])
    kc2, vc2 = oracle.swap_blocks(hk, hv, kc2, vc2, in_pairs)
    bt1, cl1 = bm2.pack(range(w.B), 8)
    got = oracle.decode(w.q, "bf16", kc2, vc2, "bf16", bt1, cl1, w.scale)
    np.testing.assert_array_equal(got, ref)
    bm2.check_invariants()


def test_swap_blocks_copies_whole_blocks_only():
    rng = np.random.default_rng(5)
    src_k = rng.integers(0, 2**16, (6, 2, 16, 8), dtype=np.uint16)
    src_v = rng.integers(0, 2**16, (6, 2, 16, 8), dtype=np.uint16)
    dst_k = np.full((4, 2, 16, 8), 7, np.uint16)
    dst_v = np.full((4, 2, 16, 8), 9, np.uint16)
    k2, v2 = oracle.swap_blocks(src_k, src_v, dst_k, dst_v, [(5, 0), (2, 3)])
    np.testing.assert_array_equal(k2[0], src_k[5])
    np.testing.assert_array_equal(v2[3], src_v[2])
    np.testing.assert_array_equal(k2[1:3], 7)
    np.testing.assert_array_equal(v2[1:3], 9)
    assert np.all(dst_k == 7)                # inputs untouched


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_invariants_hold_under_random_scripts_with_swaps(seed):
    rng = np.random.default_rng(seed)
    bm = oracle.RefBlockManager(48, free_order=rng.permutation(48), num_host_blocks=40,
                                host_free_order=rng.permutation(40))
    live, next_id = [], 0
    for _ in range(3000):
        op = rng.integers(0, 12)
        dev = [s for s in live if not bm.is_swapped(s)]
        host = [s for s in live if bm.is_swapped(s)]
        try:
            if op == 0 or not live:
                bm.add_seq(next_id)
                live.append(next_id)
                next_id += 1
            elif op == 1 and dev:
                bm.fork(int(rng.choice(dev)), next_id)
                live.append(next_id)
                next_id += 1
            elif op == 2:
                s = int(rng.choice(live))
                bm.free_seq(s)
                live.remove(s)
            elif op in (3, 4) and dev:
                k = int(rng.integers(1, min(3, len(dev)) + 1))
                group = [int(x) for x in rng.choice(dev, k, replace=False)]
                tables = {s: bm.table(s) for s in group}
                nfree_h, nfree_d = bm.num_free_host(), bm.num_free()
                pairs = bm.swap_out(group)
                distinct = {b for t in tables.values() for b in t}
                assert len(pairs) == len(distinct) == nfree_h - bm.num_free_host()
                m = dict(pairs)
                for s in group:
                    assert bm.table(s) == [m[b] for b in tables[s]]
                assert bm.num_free() >= nfree_d
            elif op == 5 and host:
                k = int(rng.integers(1, min(3, len(host)) + 1))
                group = [int(x) for x in rng.choice(host, k, replace=False)]
                tables = {s: bm.table(s) for s in group}
                pairs = bm.swap_in(group)
                m = dict(pairs)
                for s in group:
                    assert bm.table(s) == [m[b] for b in tables[s]]
            elif dev:
                s = int(rng.choice(dev))
                bm.append_tokens(s, int(rng.integers(1, 20)))
        except oracle.NoBlocks:
            pass
        bm.check_invariants()
