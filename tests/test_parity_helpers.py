"""CPU checks of the GPU tests' comparison helpers (tests/_parity.py).

* ``round_bf16`` is round-to-nearest-even to bfloat16: on values exactly
  representable in float32 it must agree with torch's float32 -> bfloat16
  conversion, and it must round float64 midpoints to even.
* The derived error bound must hold for a float32 emulation of the rounding
  steps the decode kernel takes (bf16 exponentials, float32 sums), and must
  flag a row with one position read from the wrong place.
* The q = 0 check must pass the emulated kernel's mean and flag one wrong
  position in a long context.
"""
import numpy as np
import pytest
import torch

from tests import _parity as par

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_via_torch(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(10000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(10000) * 1e20).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 2.0 ** -130], np.float32)])
    # exact float32 midpoints between neighbouring bf16 values (ties)
    bits = rng.integers(0x3F800000, 0x40800000, 5000, dtype=np.uint32)
    ties = ((bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    np.testing.assert_array_equal(par.round_bf16(x.astype(np.float64)), _bf16_via_torch(x))


def test_round_bf16_ties_to_even_in_float64():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even mantissa is 1
    assert par.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert par.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2 * 2.0 ** -7
    assert par.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert par.round_bf16(255.5) == 256.0


def test_ulp_bf16():
    assert par.ulp_bf16(1.0) == 2.0 ** -7
    assert par.ulp_bf16(1.99) == 2.0 ** -7
    assert par.ulp_bf16(0.75) == 2.0 ** -8
    assert par.ulp_bf16(-2.0) == 2.0 ** -6
    assert par.ulp_bf16(0.0) == 2.0 ** -133


def _bf16(x):
    return _bf16_via_torch(np.asarray(x, dtype=np.float32))


def _kernel_like(q, K, V, scale, tile=16):
    """float32 emulation of the decode kernel's rounding steps for one row:
    float32 logits in log2 units, running max, exponentials rounded to bf16,
    float32 sums of the rounded weights and of weight x V per 16-token tile,
    one division and one rounding to bf16 at the end."""
    x = (K.astype(np.float32) @ q.astype(np.float32)) * np.float32(scale * 1.4426950408889634)
    m = np.float32(x.max())
    p = _bf16(np.exp2((x - m).astype(np.float32))).astype(np.float32)
    l = np.float32(0)
    o = np.zeros(K.shape[1], np.float32)
    for t0 in range(0, len(x), tile):
        l = np.float32(l + p[t0:t0 + tile].sum(dtype=np.float32))
        o = (o + (p[t0:t0 + tile, None] * V[t0:t0 + tile].astype(np.float32)).sum(
            axis=0, dtype=np.float32)).astype(np.float32)
    return _bf16(o * np.float32(1.0 / l))


@pytest.mark.parametrize("L", [1, 2, 17, 300, 2048, 4096])
def test_derived_bound_holds_for_kernel_like_arithmetic(L):
    rng = np.random.default_rng(L)
    D, H = 128, 8
    scale = np.float32(1 / np.sqrt(D))
    K = _bf16(rng.standard_normal((L, D)))
    V = _bf16(rng.standard_normal((L, D)))
    Q = _bf16(rng.standard_normal((H, D)) * 3)      # sharper softmax than N(0, 1)
    got = np.stack([_kernel_like(Q[h], K, V, scale) for h in range(H)])[None]
    ref = np.zeros((1, H, D))
    for h in range(H):
        z = np.float64(scale) * (K @ Q[h])
        w = np.exp(z - z.max())
        ref[0, h] = (w / w.sum()) @ V
    S = np.abs(V[None, None] - ref[:, :, None]).max(axis=2)
    M = np.broadcast_to(np.abs(V).max(axis=0), (1, H, D))
    rec = par.check(got, ref, "bf16", f"emulated L={L}", stats=(S, M, np.array([-(-L // 16)])))
    assert rec["max_err_over_bound"] <= 1.0
    # a row that read one position from elsewhere is flagged when the
    # position carries weight
    bad = got.copy()
    h = int(np.argmax([np.max(np.exp(np.float64(scale) * (K @ Q[h]) -
                                     np.max(np.float64(scale) * (K @ Q[h])))) for h in range(H)]))
    if L > 1:
        z = np.float64(scale) * (K @ Q[h])
        w = np.exp(z - z.max())
        w /= w.sum()
        t = int(np.argmax(w))
        V2 = V.copy()
        V2[t] = V[(t + 1) % L]
        bad[0, h] = _bf16(w @ V2)
        with pytest.raises(AssertionError):
            par.check(bad, ref, "bf16", "planted", stats=(S, M, np.array([-(-L // 16)])))


@pytest.mark.parametrize("L", [700, 4096, 32768])
def test_mean_check_passes_float32_sums_and_flags_one_wrong_position(L):
    rng = np.random.default_rng(L + 1)
    D = 128
    V = _bf16(rng.standard_normal((L, D)))
    ref = V.mean(axis=0)[None, None]
    acc = np.zeros(D, np.float32)
    for t0 in range(0, L, 16):
        acc = (acc + V[t0:t0 + 16].astype(np.float32).sum(axis=0, dtype=np.float32)).astype(np.float32)
    got = _bf16(acc * np.float32(1.0 / L))[None, None]
    M = np.abs(V).max(axis=0)[None, None]
    par.check_mean_rows(got, ref, np.array([L]), M, f"emulated mean L={L}")
    V2 = V.copy()
    V2[L // 3] = V[L // 3 + 1]
    acc2 = V2.astype(np.float32).sum(axis=0, dtype=np.float32)
    bad = _bf16(acc2 * np.float32(1.0 / L))[None, None]
    with pytest.raises(AssertionError):
        par.check_mean_rows(bad, ref, np.array([L]), M, "planted")
