"""Pins of the oracle's storage formats, cache writes and block copies."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._oracle_setup import SENTINEL, empty_cache, fill_sequential, contiguous_rows


# ---------------------------------------------------------------- bf16
def test_bf16_widening_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


# ---------------------------------------------------------------- fp8 e4m3
def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e4m3_spot_values_from_the_field_definition():
    v = oracle.e4m3_all_values()
    assert v[0x7E] == 448.0                 # largest finite
    assert v[0x01] == 2.0 ** -9             # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9         # largest subnormal
    assert v[0x08] == 2.0 ** -6             # smallest normal
    assert v[0x38] == 1.0                   # exponent field 7 = bias
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0xFE] == -448.0
    # strictly increasing over the non-negative finite codes
    assert np.all(np.diff(v[:0x7F]) > 0)


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_to_f64(codes).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals, np.float32(1.0)), codes)


def test_e4m3_rounds_ties_to_even_and_nearest_otherwise():
    v = oracle.e4m3_all_values()[:0x7F]
    for c in range(0x7E):
        lo, hi = v[c], v[c + 1]
        mid = np.float32((lo + hi) / 2)        # exact: adjacent values differ in 1 bit
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]), np.float32(1))[0] == even
        assert oracle.e4m3_encode(np.array([-mid]), np.float32(1))[0] == even | 0x80
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1000))
        assert oracle.e4m3_encode(np.array([below]), np.float32(1))[0] == c
        assert oracle.e4m3_encode(np.array([above]), np.float32(1))[0] == c + 1


def test_e4m3_saturates_and_keeps_nan():
    x = np.array([448.0, 449.0, 479.9, 1e30, np.inf, -np.inf, -500.0, np.nan, -0.0, -1e-30],
                 dtype=np.float32)
    got = oracle.e4m3_encode(x, np.float32(1.0))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x80]


def test_e4m3_encode_matches_torch_in_range():
    """torch's float32 -> float8_e4m3fn conversion is round-to-nearest-even;
    it differs only past 448 (torch gives NaN, this format saturates)."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-3, 0.05, 1, 30, 150)])
    x = x[np.abs(x) < 448]
    ours = oracle.e4m3_encode(x, np.float32(1.0))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_applies_inverse_scale_in_float32():
    x = np.array([1.0, 3.0, -2.5], dtype=np.float32)
    inv = np.float32(1.0 / np.float64(np.float32(0.01)))
    got = oracle.e4m3_encode(x, inv)
    ref = oracle.e4m3_encode((x * inv).astype(np.float32), np.float32(1))
    np.testing.assert_array_equal(got, ref)
    # quantisation error is at most half a code step of the scaled value
    dec = oracle.e4m3_to_f64(got) / np.float64(inv)
    assert np.all(np.abs(dec - x) <= np.abs(x) * 2.0 ** -4 + 1e-12)


# ---------------------------------------------------------------- write_kv
@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8"])
def test_write_then_gather_returns_rows_and_keeps_sentinels(fmt):
    w = workloads.small_random(61, 3, 4, 2, 16, fmt, 50, 1)
    bm, kc, vc, bt, cl, slots = fill_sequential(w)
    written = np.zeros(kc.shape[:3], dtype=bool)
    written[slots // 16, :, slots % 16] = True
    # untouched slots keep the sentinel bit pattern
    raw = kc.view(np.uint32) if fmt == "f32" else kc
    assert np.all(raw[~written] == SENTINEL[fmt])
    for s in range(w.B):
        kr, vr = contiguous_rows(w, s)
        for g in range(w.Hkv):
            gk = oracle.gather_kv(kc, bt[s], int(cl[s]), g)
            gv = oracle.gather_kv(vc, bt[s], int(cl[s]), g)
            if fmt == "fp8":
                inv = np.float32(1.0 / np.float64(w.k_scale))
                x = workloads.bf16_bits_to_f32(kr[:, g])
                np.testing.assert_array_equal(gk, oracle.e4m3_encode(x, inv))
                # decoded back: within half a step (relative 2^-4) plus the
                # smallest subnormal step
                dec = oracle.e4m3_to_f64(gk) * np.float64(w.k_scale)
                assert np.all(np.abs(dec - x) <= np.abs(x) * 2.0 ** -4
                              + 2.0 ** -10 * np.float64(w.k_scale) + 1e-30)
            else:
                np.testing.assert_array_equal(gk.view(np.uint8), np.ascontiguousarray(kr[:, g]).view(np.uint8))
                np.testing.assert_array_equal(gv.view(np.uint8), np.ascontiguousarray(vr[:, g]).view(np.uint8))


def test_write_skips_negative_slots():
    w = workloads.small_random(62, 2, 2, 2, 8, "bf16", 20, 1)
    kc = empty_cache(w.num_blocks, w.Hkv, w.D, "bf16")
    vc = empty_cache(w.num_blocks, w.Hkv, w.D, "bf16")
    slots = -np.ones(len(w.row_seq), dtype=np.int64)
    kc2, vc2 = oracle.write_kv(kc, vc, w.k_rows, w.v_rows, slots, "bf16", "bf16")
    np.testing.assert_array_equal(kc2, kc)
    np.testing.assert_array_equal(vc2, vc)


# ---------------------------------------------------------------- copy_blocks
def test_copy_blocks_copies_whole_blocks_only():
    rng = np.random.default_rng(63)
    kc = rng.integers(0, 1 << 16, size=(10, 2, 16, 8), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(10, 2, 16, 8), dtype=np.uint16)
    pairs = [(1, 7), (4, 2), (1, 9)]
    k2, v2 = oracle.copy_blocks(kc, vc, pairs)
    for s, d in pairs:
        np.testing.assert_array_equal(k2[d], kc[s])
        np.testing.assert_array_equal(v2[d], vc[s])
    others = [b for b in range(10) if b not in (7, 2, 9)]
    np.testing.assert_array_equal(k2[others], kc[others])
    np.testing.assert_array_equal(v2[others], vc[others])


# ---------------------------------------------------------------- accounting
def test_kv_bytes_formula_on_the_long_context_shape():
    # 8 sequences x 32768 tokens x 1 layer x (8 heads x 128) x K,V x 2 bytes = 1 GiB
    assert oracle.kv_cache_bytes(8, 32768, 1, 8 * 128, 2) == 1 << 30


def test_paged_utilisation_of_the_tiny_workload():
    assert oracle.paged_utilisation([1, 15, 16, 37]) == 69 / 96
    assert oracle.paged_utilisation([16, 32]) == 1.0
