"""Pins of the oracle at block sizes other than 16 (8, 32, 64): slots and
allocation counts in closed form, copy-on-write at the new boundary,
decode from flat cache memory by the layout formula, and decode / prefix
caching equal to the 16-token case on the same rows."""
import numpy as np
import pytest

import oracle
import workloads
from tests.test_oracle_attention import _decimal_attention


def _fill(w, bs, kv_fmt="f32"):
    """The workload's rows written through a manager of block size bs."""
    nb = sum(-(-int(L) // bs) for L in w.lens) + 4
    bm = oracle.RefBlockManager(nb, block_size=bs, free_order=np.random.default_rng(bs).permutation(nb))
    per = {}
    for s in range(w.B):
        bm.add_seq(s)
        per[s], pair = bm.append_tokens(s, int(w.lens[s]))
        assert pair is None
    slots = np.array([per[int(s)][int(p)] for s, p in zip(w.row_seq, w.row_pos)], np.int64)
    dt = np.float32 if kv_fmt == "f32" else np.uint16
    kc = np.zeros((nb, w.Hkv, bs, w.D), dt)
    vc = np.zeros_like(kc)
    kc, vc = oracle.write_kv(kc, vc, w.k_rows, w.v_rows, slots, w.src_fmt, w.fmt)
    cap = max(-(-int(L) // bs) for L in w.lens)
    bt, cl = bm.pack(list(range(w.B)), cap)
    return bm, kc, vc, bt, cl


@pytest.mark.parametrize("bs", [8, 32, 64])
def test_slots_and_block_counts_closed_form(bs):
    bm = oracle.RefBlockManager(40, block_size=bs)
    bm.add_seq(0)
    slots, _ = bm.append_tokens(0, 3 * bs + 5)
    t = bm.table(0)
    assert len(t) == 4 and t == [0, 1, 2, 3]
    assert slots == [t[p // bs] * bs + p % bs for p in range(3 * bs + 5)]
    assert bm.num_free() == 36
    with pytest.raises(ValueError):
        oracle.RefBlockManager(4, block_size=24)


@pytest.mark.parametrize("bs", [8, 32])
def test_copy_on_write_at_the_block_size(bs):
    bm = oracle.RefBlockManager(10, block_size=bs)
    bm.add_seq(0)
    bm.append_tokens(0, bs + 3)                   # block 1 partial
    bm.fork(0, 1)
    slot, pair = bm.append_slot(1)
    assert pair == (1, 2) and slot == 2 * bs + 3
    bm.add_seq(2)
    bm.append_tokens(2, bs)                       # exactly one full block
    bm.fork(2, 3)
    slot, pair = bm.append_slot(3)                # a new block, no copy
    assert pair is None and slot == bm.table(3)[1] * bs


@pytest.mark.parametrize("bs", [8, 32, 64])
def test_decode_matches_decimal_brute_force_at_block_size(bs):
    w = workloads.small_random(40 + bs, 3, 4, 2, 8, "f32", 70, 1)
    bm, kc, vc, bt, cl = _fill(w, bs)
    out = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    fk, fv = kc.reshape(-1), vc.reshape(-1)
    for s in range(w.B):
        L = int(cl[s])
        for h in range(w.Hq):
            g = h // 2
            idx = [((bt[s, t // bs] * w.Hkv + g) * bs + t % bs) * w.D for t in range(L)]
            K = [[fk[i + d] for d in range(w.D)] for i in idx]
            V = [[fv[i + d] for d in range(w.D)] for i in idx]
            np.testing.assert_allclose(out[s, h], _decimal_attention(w.q[s, h], K, V, w.scale),
                                       rtol=0, atol=1e-14)


@pytest.mark.parametrize("bs", [8, 32, 64])
def test_decode_is_independent_of_block_size(bs):
    w = workloads.small_random(50, 5, 8, 2, 16, "bf16", 150, 1)
    _, kc16, vc16, bt16, cl16 = _fill(w, 16, "bf16")
    _, kc, vc, bt, cl = _fill(w, bs, "bf16")
    a = oracle.decode(w.q, "bf16", kc16, vc16, "bf16", bt16, cl16, w.scale)
    b = oracle.decode(w.q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    np.testing.assert_array_equal(a, b)


def test_prefix_caching_shares_whole_blocks_of_the_block_size():
    bm = oracle.RefBlockManager(20, block_size=32)
    bm.enable_prefix_caching()
    bm.add_seq_prompt(0, list(range(70)))         # 2 full blocks of 32
    slots, nc = bm.add_seq_prompt(1, list(range(64)) + [9])
    assert nc == 64 and bm.table(1)[:2] == bm.table(0)[:2]
    slots, nc = bm.add_seq_prompt(2, list(range(40)))
    assert nc == 32                               # a 16-token match is not a block


def test_paged_utilisation_depends_on_block_size():
    lens = [1, 16, 17, 40]
    assert oracle.paged_utilisation(lens, 8) == 74 / 88       # 1 + 2 + 3 + 5 blocks
    assert oracle.paged_utilisation(lens) == 74 / 112
    assert oracle.paged_utilisation(lens, 64) == 74 / 256
