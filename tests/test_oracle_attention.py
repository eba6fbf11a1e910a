"""Pins of the oracle's decode attention to things other than itself.

Each test is chosen so that a plausible slip in ``oracle.decode`` (a wrong
gather index, a dropped scale, a transposed operand, a wrong GQA head map, a
missing max subtraction, an off-by-one in the length) fails at least one of
them: 50-digit brute force, a library routine, closed forms, invariants.
"""
import decimal
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._oracle_setup import (contiguous_rows, empty_cache, fill_sequential)


def _tiny(seed, fmt="f32", B=3, Hq=4, Hkv=2, D=8, max_len=40, min_len=1, lens=None):
    return workloads.small_random(seed, B, Hq, Hkv, D, fmt, max_len, min_len, lens=lens)


def _src64(rows, fmt):
    if fmt == "f32":
        return np.asarray(rows, dtype=np.float64)
    return oracle.bf16_to_f64(rows)


# ---------------------------------------------------------------- brute force
def _decimal_attention(q, K, V, scale):
    """softmax(scale q.K^T) V with 50-digit decimals, explicit loops and no
    max subtraction (the textbook form, exp of the raw logits)."""
    ctx = decimal.Context(prec=50)
    Dc = lambda x: ctx.create_decimal(repr(float(x)))
    sc = Dc(scale)
    z = [ctx.multiply(sc, sum((ctx.multiply(Dc(q[d]), Dc(K[t][d])) for d in range(len(q))),
                              decimal.Decimal(0))) for t in range(len(K))]
    e = [ctx.exp(x) for x in z]
    tot = sum(e, decimal.Decimal(0))
    return [float(sum((ctx.multiply(e[t] / tot, Dc(V[t][d])) for t in range(len(K))),
                      decimal.Decimal(0))) for d in range(len(V[0]))]


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_decode_matches_decimal_brute_force_from_flat_memory(seed):
    """The brute force reads K/V from the flat cache memory with the layout
    formula ((b*Hkv + g)*16 + t)*D + d, walking the block table by hand."""
    w = _tiny(seed)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    flatk, flatv = kc.reshape(-1), vc.reshape(-1)
    G = w.Hq // w.Hkv
    for s in range(w.B):
        L = int(cl[s])
        for h in range(w.Hq):
            g = h // G
            K = [[flatk[((bt[s, t // 16] * w.Hkv + g) * 16 + t % 16) * w.D + d]
                  for d in range(w.D)] for t in range(L)]
            V = [[flatv[((bt[s, t // 16] * w.Hkv + g) * 16 + t % 16) * w.D + d]
                  for d in range(w.D)] for t in range(L)]
            ref = _decimal_attention(w.q[s, h], K, V, w.scale)
            np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("fmt,seed,G", [("f32", 21, 1), ("f32", 22, 4), ("bf16", 23, 4),
                                        ("bf16", 24, 8)])
def test_decode_matches_torch_sdpa_on_generator_rows(fmt, seed, G):
    """torch scaled_dot_product_attention (CPU, float64) over the contiguous
    rows exactly as the generator produced them -- no block table, no cache --
    pins write_kv + block manager + gather + attention together."""
    Hkv = 2
    w = workloads.small_random(seed, 5, Hkv * G, Hkv, 64, fmt, 100, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, w.q_fmt, kc, vc, w.fmt, bt, cl, w.scale)
    q64 = _src64(w.q, w.fmt)
    for s in range(w.B):
        kr, vr = contiguous_rows(w, s)
        K = torch.from_numpy(_src64(kr, w.fmt)).permute(1, 0, 2)       # [Hkv, L, D]
        V = torch.from_numpy(_src64(vr, w.fmt)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).unsqueeze(0)
        V = V.repeat_interleave(G, dim=0).unsqueeze(0)
        q = torch.from_numpy(q64[s]).unsqueeze(0).unsqueeze(2)          # [1, Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, K, V, scale=float(w.scale)).squeeze(2).squeeze(0).numpy()
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_of_values():
    w = _tiny(31, lens=np.array([5, 16, 33]))
    w.q[:] = 0.0
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    for s in range(w.B):
        _, vr = contiguous_rows(w, s)
        mean = np.asarray(vr, np.float64).mean(axis=0)              # [Hkv, D]
        np.testing.assert_allclose(out[s], np.repeat(mean, 2, axis=0), atol=1e-15)


def test_equal_value_rows_return_that_row():
    w = _tiny(32, lens=np.array([7, 20, 40]))
    row = np.linspace(-1, 1, w.D).astype(np.float32)
    w.v_rows[:] = row
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=0, atol=1e-15)


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_single_token_context_returns_its_value_row_exactly(fmt):
    w = workloads.small_random(33, 4, 4, 2, 64, fmt, 1, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, w.q_fmt, kc, vc, w.fmt, bt, cl, w.scale)
    for s in range(w.B):
        _, vr = contiguous_rows(w, s)
        np.testing.assert_array_equal(out[s], np.repeat(_src64(vr[0], fmt), 2, axis=0))


def test_two_token_softmax_weights_closed_form():
    """Logits 0 and ln 2 give weights 1/3 and 2/3: out = (v0 + 2 v1) / 3."""
    D = 4
    w = _tiny(34, B=1, Hq=1, Hkv=1, D=D, lens=np.array([2]))
    w.k_rows[:] = 0.0
    w.k_rows[1, 0, 0] = np.float32(1.0)
    w.q[:] = 0.0
    w.q[0, 0, 0] = np.float32(math.log(2.0))
    w.scale = np.float32(1.0)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out, wts = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale, want_weights=True)
    lg = np.float64(np.float32(math.log(2.0)))
    exp_w = np.array([1.0, math.exp(lg)]) / (1.0 + math.exp(lg))
    np.testing.assert_allclose(wts[(0, 0)], exp_w, rtol=0, atol=1e-16)
    v = np.asarray(w.v_rows[:, 0], np.float64)
    np.testing.assert_allclose(out[0, 0], exp_w[0] * v[0] + exp_w[1] * v[1], atol=1e-15)


def test_zero_context_gives_zero_row():
    w = _tiny(35, lens=np.array([0, 3, 0]))
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isfinite(out[1]))


# ---------------------------------------------------------------- invariants
def test_weights_sum_to_one_and_output_in_convex_hull():
    w = workloads.small_random(41, 6, 8, 2, 32, "bf16", 300, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out, wts = oracle.decode(w.q, "bf16", kc, vc, "bf16", bt, cl, w.scale, want_weights=True)
    for (s, h), wt in wts.items():
        assert abs(wt.sum() - 1.0) < 1e-12
        assert np.all(wt >= 0)
        _, vr = contiguous_rows(w, s)
        V = oracle.bf16_to_f64(vr)[:, h // 4]
        assert np.all(out[s, h] <= V.max(axis=0) + 1e-12)
        assert np.all(out[s, h] >= V.min(axis=0) - 1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    G = 4
    w = workloads.small_random(42, 3, 2 * G, 2, 16, "f32", 70, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out_gqa = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    kc_m = np.repeat(kc, G, axis=1)
    vc_m = np.repeat(vc, G, axis=1)
    out_mha = oracle.decode(w.q, "f32", kc_m, vc_m, "f32", bt, cl, w.scale)
    np.testing.assert_array_equal(out_gqa, out_mha)


def test_head_mapping_is_contiguous_groups():
    """Query head h reads KV head h // G: zeroing V of KV head 1 zeroes query
    heads G..2G-1 and nothing else."""
    G = 3
    w = workloads.small_random(43, 2, 2 * G, 2, 8, "f32", 30, 1)
    w.v_rows[:, 1, :] = 0.0
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    assert np.all(out[:, G:] == 0)
    assert np.all(np.abs(out[:, :G]).sum(axis=-1) > 0)


@pytest.mark.parametrize("part", [16, 48, 512])
def test_partitioned_merge_equals_unpartitioned(part):
    w = workloads.small_random(44, 4, 4, 2, 32, "bf16", 1500, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    a = oracle.decode(w.q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    b = oracle.decode_partitioned(w.q, "bf16", kc, vc, "bf16", bt, cl, w.scale, partition=part)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_merge_of_one_partition_is_identity_and_handles_far_maxima():
    o = np.random.default_rng(0).standard_normal((1, 8))
    np.testing.assert_array_equal(oracle.merge_partitions(np.array([3.0]), np.array([2.5]), o), o[0])
    # a partition whose max is 800 below the other contributes exp(-800) = 0
    o2 = np.stack([o[0], -o[0]])
    r = oracle.merge_partitions(np.array([0.0, -800.0]), np.array([1.0, 1.0]), o2)
    np.testing.assert_array_equal(r, o[0])


# ---------------------------------------------------------------- gather / layout
def test_physical_block_permutation_is_bit_invariant():
    w = workloads.small_random(51, 5, 8, 2, 64, "bf16", 200, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode(w.q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    pi = np.random.default_rng(5).permutation(w.num_blocks)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1)
    out2 = oracle.decode(w.q, "bf16", kc2, vc2, "bf16", bt2, cl, w.scale)
    np.testing.assert_array_equal(out, out2)


def test_identity_table_gather_is_a_reshape():
    rng = np.random.default_rng(52)
    nb, Hkv, D = 6, 2, 8
    cache = rng.standard_normal((nb, Hkv, 16, D))
    bt = np.arange(nb)
    for L in [1, 16, 17, 96]:
        for g in range(Hkv):
            got = oracle.gather_kv(cache, bt, L, g)
            ref = cache[:, g].reshape(nb * 16, D)[:L]
            np.testing.assert_array_equal(got, ref)


def test_unused_slots_and_table_padding_are_never_read():
    w = workloads.small_random(53, 4, 4, 2, 32, "bf16", 70, 1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w, cap=12)
    out = oracle.decode(w.q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    # every never-written slot is already a NaN sentinel; also point padding at
    # a block full of NaN and check nothing changes
    assert np.all(bt[:, -1] == -1)
    kc2 = np.concatenate([kc, empty_cache(1, w.Hkv, w.D, "bf16")])
    vc2 = np.concatenate([vc, empty_cache(1, w.Hkv, w.D, "bf16")])
    bt2 = np.where(bt < 0, w.num_blocks, bt)
    out2 = oracle.decode(w.q, "bf16", kc2, vc2, "bf16", bt2, cl, w.scale)
    assert np.all(np.isfinite(out))
    np.testing.assert_array_equal(out, out2)


def test_decode_detects_a_planted_transpose():
    """Sanity of the pins themselves: an attention with K and V swapped (a
    plausible slip) disagrees with the library routine."""
    w = workloads.small_random(54, 2, 2, 2, 16, "f32", 40, 5)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    wrong = oracle.decode(w.q, "f32", vc, kc, "f32", bt, cl, w.scale)
    right = oracle.decode(w.q, "f32", kc, vc, "f32", bt, cl, w.scale)
    assert np.abs(wrong - right).max() > 1e-3
