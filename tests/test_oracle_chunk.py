"""Pins of the oracle's chunk attention (T new tokens per sequence, causal
within the chunk) to things other than itself.

A plausible slip -- an off-by-one in the visible length, a token attending a
later chunk token, a wrong q row for a chunk token, a missing zero rule --
fails at least one of: 50-digit brute force from flat cache memory, torch's
scaled_dot_product_attention with an explicit causal mask, T successive
single-token decodes, and the no-leak / zero-row invariants.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.chunk
import workloads
from tests._oracle_setup import contiguous_rows, fill_sequential
from tests.test_oracle_attention import _decimal_attention, _src64


def _chunk_case(seed, fmt="f32", B=3, Hq=4, Hkv=2, D=8, T=3, max_len=40, min_len=1,
                lens=None):
    w = workloads.small_random(seed, B, Hq, Hkv, D, fmt, max_len, min_len, lens=lens)
    rng = np.random.default_rng(seed + 1000)
    q = workloads.chunk_queries(rng, B, T, Hq, D, fmt)
    return w, q


@pytest.mark.parametrize("seed", [61, 62])
def test_chunk_matches_decimal_brute_force_from_flat_memory(seed):
    T = 3
    w, q = _chunk_case(seed, T=T, lens=np.array([1, 3, 21]))
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale)
    flatk, flatv = kc.reshape(-1), vc.reshape(-1)
    G = w.Hq // w.Hkv
    for s in range(w.B):
        L = int(cl[s])
        for i in range(T):
            pos = L - T + i                     # position of chunk token i
            for h in range(w.Hq):
                g = h // G
                if pos < 0:
                    np.testing.assert_array_equal(out[s, i, h], 0.0)
                    continue
                K = [[flatk[((bt[s, t // 16] * w.Hkv + g) * 16 + t % 16) * w.D + d]
                      for d in range(w.D)] for t in range(pos + 1)]
                V = [[flatv[((bt[s, t // 16] * w.Hkv + g) * 16 + t % 16) * w.D + d]
                      for d in range(w.D)] for t in range(pos + 1)]
                ref = _decimal_attention(q[s, i, h], K, V, w.scale)
                np.testing.assert_allclose(out[s, i, h], ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("fmt,seed,G,T", [("f32", 71, 1, 16), ("f32", 72, 4, 4),
                                          ("bf16", 73, 4, 5), ("bf16", 74, 8, 2)])
def test_chunk_matches_torch_sdpa_with_causal_mask(fmt, seed, G, T):
    """SDPA (CPU, float64) over the generator's contiguous rows, with the
    boolean mask [T, L]: chunk token i may see position t iff t <= L - T + i."""
    Hkv = 2
    w = workloads.small_random(seed, 4, Hkv * G, Hkv, 64, fmt, 90, T)
    q = workloads.chunk_queries(np.random.default_rng(seed), w.B, T, w.Hq, w.D, fmt)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, w.q_fmt, kc, vc, w.fmt, bt, cl, w.scale)
    q64 = _src64(q, fmt)
    for s in range(w.B):
        L = int(cl[s])
        kr, vr = contiguous_rows(w, s)
        K = torch.from_numpy(_src64(kr, fmt)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(_src64(vr, fmt)).permute(1, 0, 2).repeat_interleave(G, 0)
        Q = torch.from_numpy(q64[s]).permute(1, 0, 2)                  # [Hq, T, D]
        mask = torch.arange(L)[None, :] <= (L - T + torch.arange(T))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0), attn_mask=mask,
            scale=float(w.scale)).squeeze(0).permute(1, 0, 2).numpy()   # [T, Hq, D]
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [1, 2, 7])
def test_chunk_rows_equal_successive_single_token_decodes(T):
    """Chunk token i gives what a decode step at context length L - T + i + 1
    gives with the same cache and table (the chunk is T decode steps in one)."""
    w, q = _chunk_case(81, fmt="bf16", B=5, Hq=8, Hkv=2, D=16, T=T, max_len=70)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    for i in range(T):
        cl_i = np.maximum(cl - T + i + 1, 0).astype(np.int32)
        ref = oracle.decode(q[:, i], "bf16", kc, vc, "bf16", bt, cl_i, w.scale)
        np.testing.assert_allclose(out[:, i], ref, rtol=0, atol=1e-15)


def test_chunk_of_one_token_is_decode():
    w, q = _chunk_case(82, fmt="f32", T=1)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale)
    ref = oracle.decode(q[:, 0], "f32", kc, vc, "f32", bt, cl, w.scale)
    np.testing.assert_array_equal(out[:, 0], ref)


def test_later_positions_never_leak_into_earlier_chunk_tokens():
    """Changing the cache rows of positions after chunk token i's own position
    leaves token i's output bit-identical, while the tokens that see those
    positions change: V rows set to 1e6 move them by far more than 1, K rows
    set to NaN make them NaN."""
    T = 4
    w, q = _chunk_case(83, fmt="f32", B=2, T=T, lens=np.array([19, 35]))
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale)
    for s in range(w.B):
        L = int(cl[s])
        for i in range(T - 1):
            later = [(bt[s, t // 16], t % 16) for t in range(L - T + i + 1, L)]
            vc2 = vc.copy()
            kc3 = kc.copy()
            for b, o in later:
                vc2[b, :, o, :] = 1e6
                kc3[b, :, o, :] = np.nan
            out2 = oracle.decode_chunk(q, "f32", kc, vc2, "f32", bt, cl, w.scale)
            np.testing.assert_array_equal(out2[s, :i + 1], out[s, :i + 1])
            assert np.abs(out2[s, i + 1:] - out[s, i + 1:]).min(axis=-1).min() > 1.0
            out3 = oracle.decode_chunk(q, "f32", kc3, vc, "f32", bt, cl, w.scale)
            np.testing.assert_array_equal(out3[s, :i + 1], out[s, :i + 1])
            assert np.all(np.isnan(out3[s, i + 1:]))


def test_tokens_without_visible_positions_get_zero_rows():
    """L < T: chunk tokens i < T - L see nothing (zero rows); the rest see
    positions 0 .. i - (T - L)."""
    T = 6
    w, q = _chunk_case(84, fmt="f32", B=3, T=T, lens=np.array([0, 2, 6]))
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale)
    np.testing.assert_array_equal(out[0], 0.0)
    np.testing.assert_array_equal(out[1, :4], 0.0)
    assert np.all(np.abs(out[1, 4:]).max(axis=-1) > 0)
    # token T - L of the L = 2 sequence sees position 0 only: its V row
    _, vr = contiguous_rows(w, 1)
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        np.testing.assert_array_equal(out[1, 4, h], np.float64(vr[0, h // G]))
    assert np.all(np.isfinite(out))


def test_sampled_rows_equal_the_full_chunk_oracle():
    T = 5
    w, q = _chunk_case(85, fmt="bf16", B=4, Hq=8, Hkv=2, D=16, T=T, max_len=50)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    full = oracle.decode_chunk(q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    picks = [(0, 0, 0), (1, 4, 7), (2, 2, 3), (3, 1, 5)]
    rows = oracle.chunk_rows(q, "bf16", kc, vc, "bf16", bt, cl, w.scale, picks=picks)
    for r, (s, i, h) in zip(rows, picks):
        np.testing.assert_array_equal(r, full[s, i, h])


def test_pins_catch_a_planted_off_by_one_in_the_visible_length(monkeypatch):
    """Sanity of the pins: an oracle whose chunk tokens see one position too
    few disagrees with the masked library attention."""
    T, G = 3, 2
    w = workloads.small_random(86, 2, 4, 2, 16, "f32", 40, T + 1)
    q = workloads.chunk_queries(np.random.default_rng(86), w.B, T, w.Hq, w.D, "f32")
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    right = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale)
    monkeypatch.setattr(oracle.chunk, "visible_len",
                        lambda L, T_, i: max(0, int(L) - int(T_) + int(i)))
    wrong = oracle.chunk.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale)
    assert np.abs(wrong - right).max() > 1e-3


# ---------------------------------------------------------------- sliding window
@pytest.mark.parametrize("W,T", [(1, 1), (5, 1), (17, 3), (40, 4), (1000, 2)])
def test_window_matches_torch_sdpa_with_band_mask(W, T):
    """SDPA over the generator's rows with the band mask: chunk token i (at
    position p = L - T + i) sees t iff p - W < t <= p."""
    G = 2
    w = workloads.small_random(90 + W, 4, 4, 2, 32, "f32", 120, T)
    q = workloads.chunk_queries(np.random.default_rng(W), w.B, T, w.Hq, w.D, "f32")
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale, window=W)
    for s in range(w.B):
        L = int(cl[s])
        kr, vr = contiguous_rows(w, s)
        K = torch.from_numpy(np.asarray(kr, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(np.asarray(vr, np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
        Q = torch.from_numpy(np.asarray(q[s], np.float64)).permute(1, 0, 2)
        p = (L - T + torch.arange(T))[:, None]
        t = torch.arange(L)[None, :]
        mask = (t <= p) & (t > p - W)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0), attn_mask=mask,
            scale=float(w.scale)).squeeze(0).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


def test_window_of_one_returns_the_tokens_own_value_row():
    T = 3
    w, q = _chunk_case(91, fmt="f32", T=T, lens=np.array([3, 20, 33]))
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    out = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale, window=1)
    G = w.Hq // w.Hkv
    for s in range(w.B):
        _, vr = contiguous_rows(w, s)
        for i in range(T):
            p = int(cl[s]) - T + i
            for h in range(w.Hq):
                np.testing.assert_array_equal(out[s, i, h], np.float64(vr[p, h // G]))


def test_window_covering_the_context_changes_nothing_and_sampled_rows_agree():
    T = 2
    w, q = _chunk_case(92, fmt="bf16", B=4, Hq=8, Hkv=2, D=16, T=T, max_len=60)
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    full = oracle.decode_chunk(q, "bf16", kc, vc, "bf16", bt, cl, w.scale)
    wide = oracle.decode_chunk(q, "bf16", kc, vc, "bf16", bt, cl, w.scale, window=60)
    np.testing.assert_array_equal(full, wide)
    narrow = oracle.decode_chunk(q, "bf16", kc, vc, "bf16", bt, cl, w.scale, window=9)
    picks = [(0, 0, 0), (1, 1, 7), (3, 0, 2)]
    rows = oracle.chunk_rows(q, "bf16", kc, vc, "bf16", bt, cl, w.scale, picks=picks, window=9)
    for r, (s, i, h) in zip(rows, picks):
        np.testing.assert_array_equal(r, narrow[s, i, h])


def test_pins_catch_a_planted_off_by_one_in_the_window(monkeypatch):
    T, W = 2, 7
    w = workloads.small_random(93, 3, 4, 2, 16, "f32", 50, 20)
    q = workloads.chunk_queries(np.random.default_rng(93), w.B, T, w.Hq, w.D, "f32")
    bm, kc, vc, bt, cl, _ = fill_sequential(w)
    right = oracle.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale, window=W)
    monkeypatch.setattr(oracle.chunk, "window_start",
                        lambda n, window: max(0, int(n) - int(window) + 1))
    wrong = oracle.chunk.decode_chunk(q, "f32", kc, vc, "f32", bt, cl, w.scale, window=W)
    assert np.abs(wrong - right).max() > 1e-3
