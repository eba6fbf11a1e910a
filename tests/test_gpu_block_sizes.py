"""GPU parity at block sizes 8, 32 and 64 through the C ABI: the library's
slots and cache bytes equal the oracle's bit for bit, copy-on-write copies
are exact, and decode / chunks / windows match the oracle.  32- and 64-token
blocks stream as 2 or 4 tiles of 16, 8-token blocks as tiles of two blocks;
an fp32 cache takes the partition path at every block size; 8-token blocks in a
cache over 2 GiB give the small cache's results bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import _oracle_setup as osu
from tests._gpu_setup import cache_to_numpy, out_to_f64, to_device_rows, TORCH_STORE, TORCH_VIEW

pk = pytest.importorskip("paged_kv_cache_421_amd")

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def _say(msg):
    print(msg, flush=True)


def _cache(nb, w, bs):
    val = int(osu.SENTINEL[w.fmt])
    if w.fmt == "f32":
        val = val - (1 << 32) if val >= (1 << 31) else val
    return torch.full((nb, w.Hkv, bs, w.D), val, dtype=TORCH_STORE[w.fmt],
                      device="cuda").view(TORCH_VIEW[w.fmt])


def _oracle_cache(nb, w, bs):
    if w.fmt == "f32":
        return np.full((nb, w.Hkv, bs, w.D), osu.SENTINEL["f32"], np.uint32).view(np.float32)
    return np.full((nb, w.Hkv, bs, w.D), osu.SENTINEL[w.fmt], osu.STORE[w.fmt])


def _build(seed, fmt, bs, G, D, lens, Hkv=2):
    w = workloads.small_random(seed, len(lens), G * Hkv, Hkv, D, fmt, 0, lens=np.asarray(lens, np.int32))
    nb = sum(-(-int(L) // bs) for L in w.lens) + 3
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    poison = nb                                   # never allocated, stays NaN
    ref = oracle.RefBlockManager(nb, free_order=order, block_size=bs)
    lib = pk.BlockManager(nb, free_order=order, block_size=bs)
    per_r, per_l = {}, {}
    for s in range(w.B):
        ref.add_seq(s)
        lib.add_seq(s)
        per_r[s], _ = ref.append_tokens(s, int(w.lens[s]))
        per_l[s], _ = lib.append_tokens(s, int(w.lens[s]))
        assert list(per_l[s]) == per_r[s]
    slots = np.array([per_r[int(s)][int(p)] for s, p in zip(w.row_seq, w.row_pos)], np.int64)
    desc = pk.CacheDesc(nb + 1, Hkv, D, fmt, w.k_scale, w.v_scale, block_size=bs)
    kc, vc = _cache(nb + 1, w, bs), _cache(nb + 1, w, bs)
    if len(slots):
        pk.write_kv(desc, kc, vc, to_device_rows(w.k_rows, w.src_fmt), to_device_rows(w.v_rows, w.src_fmt),
                    torch.from_numpy(slots).cuda())
    kc_o, vc_o = oracle.write_kv(_oracle_cache(nb + 1, w, bs), _oracle_cache(nb + 1, w, bs),
                                 w.k_rows, w.v_rows, slots, w.src_fmt, w.fmt, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(cache_to_numpy(kc, fmt).view(np.uint8), kc_o.view(np.uint8))
    assert np.array_equal(cache_to_numpy(vc, fmt).view(np.uint8), vc_o.view(np.uint8))
    cap = max(1, max(-(-int(L) // bs) for L in w.lens))
    bt, cl = ref.pack(list(range(w.B)), cap)
    bt = np.where(bt < 0, poison, bt).astype(np.int32)
    return w, desc, kc, vc, kc_o, vc_o, bt, cl


LENS = [0, 1, 7, 8, 9, 31, 32, 33, 64, 65, 200, 513, 1100]


@pytest.mark.parametrize("bs,fmt,G,D", [(8, "bf16", 4, 128), (32, "bf16", 4, 128),
                                        (64, "bf16", 8, 64), (32, "fp8", 4, 128),
                                        (64, "f32", 2, 64), (8, "fp8", 2, 64),
                                        (8, "f32", 2, 128), (8, "bf16", 16, 64), (8, "fp8", 4, 128)])
def test_decode_chunk_and_window_at_block_size(bs, fmt, G, D):
    w, desc, kc, vc, kc_o, vc_o, bt, cl = _build(1000 + bs + D, fmt, bs, G, D, LENS)
    _say(f"block size {bs} {fmt} G={G} D={D}")
    btd = torch.from_numpy(bt).cuda()
    cld = torch.from_numpy(cl).cuda()
    max_len = int(cl.max())
    for T, W in ((1, 0), (4, 0), (3, 40)):
        q = workloads.chunk_queries(np.random.default_rng(bs + T + W), w.B, T, w.Hq, D, w.q_fmt)
        qd = to_device_rows(q, w.q_fmt)
        out = torch.empty_like(qd)
        pk.decode_chunk(desc, kc, vc, qd, out, btd, cld, max_len, float(w.scale), window=W)
        torch.cuda.synchronize()
        ref = oracle.decode_chunk(q, w.q_fmt, kc_o, vc_o, fmt, bt, cl, w.scale, w.k_scale,
                                  w.v_scale, window=W)
        got = out_to_f64(out)
        assert np.all(np.isfinite(got))
        err = np.abs(got - ref).max()
        assert err <= TOL[fmt], (T, W, err)
        _say(f"  T={T} W={W}: max abs err {err:.3e}")


@pytest.mark.parametrize("bs", [8, 32])
def test_copy_on_write_at_block_size(bs):
    w, desc, kc, vc, kc_o, vc_o, bt, cl = _build(1100 + bs, "bf16", bs, 4, 128, [bs + 5, 3 * bs])
    nb = desc.c.num_blocks - 1
    lib = pk.BlockManager(nb, block_size=bs)
    ref = oracle.RefBlockManager(nb, block_size=bs)
    for m in (lib, ref):
        m.add_seq(0)
        m.append_tokens(0, bs + 5)
        m.fork(0, 1)
    _, pair = lib.append_slot(1)
    _, rpair = ref.append_slot(1)
    assert tuple(pair) == rpair
    p = torch.tensor([list(pair)], dtype=torch.int32, device="cuda")
    pk.copy_blocks(desc, kc, vc, p)
    kc_o, vc_o = oracle.copy_blocks(kc_o, vc_o, [rpair])
    torch.cuda.synchronize()
    assert np.array_equal(cache_to_numpy(kc, "bf16").view(np.uint8), kc_o.view(np.uint8))
    assert np.array_equal(cache_to_numpy(vc, "bf16").view(np.uint8), vc_o.view(np.uint8))


@pytest.mark.parametrize("fmt,G,D", [("bf16", 4, 128), ("fp8", 8, 64)])
def test_8_token_blocks_in_caches_over_2gib(fmt, G, D):
    """Caches of 2 GiB and more cannot be addressed by one buffer descriptor
    with 32-bit offsets, so their 8-token tiles take a descriptor per block.
    The small case's blocks are placed in a 2.5 GiB cache, every other one
    past 2 GiB (so tiles straddle the boundary): decode, chunks and windows
    give the small cache's results bit for bit (those match the oracle in
    test_decode_chunk_and_window_at_block_size)."""
    bs = 8
    w, desc, kc, vc, kc_o, vc_o, bt, cl = _build(1200 + D, fmt, bs, G, D, LENS)
    nb = desc.c.num_blocks
    per_block = w.Hkv * bs * D * (1 if fmt == "fp8" else 2)
    nb_big = (5 << 29) // per_block                       # 2.5 GiB per cache
    high = (1 << 31) // per_block + 1000                  # first block id past 2 GiB
    ids = np.arange(nb)
    to_big = np.where(ids % 2 == 0, ids, high + ids).astype(np.int64)
    assert to_big.max() < nb_big
    desc_big = pk.CacheDesc(nb_big, w.Hkv, D, fmt, w.k_scale, w.v_scale, block_size=bs)
    kb = torch.zeros((nb_big, w.Hkv, bs, D), dtype=kc.dtype, device="cuda")
    vb = torch.zeros_like(kb)
    idx = torch.from_numpy(to_big).cuda()
    kb.index_copy_(0, idx, kc)
    vb.index_copy_(0, idx, vc)
    bt_big = to_big[bt].astype(np.int32)
    _say(f"8-token blocks {fmt} G={G} D={D}: cache {nb_big} blocks, {nb_big * per_block / 2**30:.2f} GiB")
    cld = torch.from_numpy(cl).cuda()
    max_len = int(cl.max())
    for T, W in ((1, 0), (4, 0), (3, 40)):
        q = workloads.chunk_queries(np.random.default_rng(bs + T + W), w.B, T, w.Hq, D, w.q_fmt)
        qd = to_device_rows(q, w.q_fmt)
        small, big = torch.empty_like(qd), torch.empty_like(qd)
        pk.decode_chunk(desc, kc, vc, qd, small, torch.from_numpy(bt).cuda(), cld, max_len,
                        float(w.scale), window=W)
        pk.decode_chunk(desc_big, kb, vb, qd, big, torch.from_numpy(bt_big).cuda(), cld, max_len,
                        float(w.scale), window=W)
        torch.cuda.synchronize()
        assert torch.equal(small.view(torch.int16), big.view(torch.int16)), (T, W)
        _say(f"  T={T} W={W}: bit-identical")
    del kb, vb
    torch.cuda.empty_cache()
