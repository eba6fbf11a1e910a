"""Storage formats of the KV cache, decoded from their definitions (oracle).

* float32: IEEE binary32, stored as is.
* bfloat16: the upper 16 bits of a binary32 (sign, 8-bit exponent, 7-bit
  mantissa); widening appends 16 zero bits, so it is exact.
* fp8 E4M3 ("e4m3fn" in the OCP 8-bit floating point specification): sign bit,
  4-bit exponent with bias 7, 3-bit mantissa; no infinities; exponent 15 with
  mantissa 7 is NaN; exponent 0 encodes subnormals ``m * 2**-9``; the largest
  finite magnitude is 448.

The pages name FP8 only as a quantisation format supported by the engine
(explore.n1n.ai, "vLLM 深度解析", feature list; ybb.press, "vLLM
PagedAttention 大模型推理架构深度实战", §5.2).  Which FP8 variant, how it is
rounded and how it is scaled are not on the pages; the readings used here are:
E4M3 as above, one float32 scale per cache tensor, stored value =
code value x scale, and quantisation code = round-to-nearest-even of
``sat448(fp32(x * fp32(1/scale)))``, keeping the sign of the scaled value
(negative values that round to zero give the negative-zero code 0x80, NaN gives
0x7F).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):     # NaN payloads widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """Value of one E4M3 code, straight from the field definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_all_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    return _E4M3_TABLE.copy()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 codes (uint8) to float64."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_VALUES = _E4M3_TABLE[:0x7F]


def e4m3_encode(x: np.ndarray, inv_scale: np.float32) -> np.ndarray:
    """Quantise float32 values to E4M3 codes.

    y = fp32(x * inv_scale) (one float32 multiply, round-to-nearest-even);
    NaN -> 0x7F; |y| >= 448 (infinities included) -> 448 with y's sign;
    otherwise the representable magnitude nearest to |y|, ties going to the
    code with an even mantissa, with y's sign bit.
    """
    xf = np.asarray(x, dtype=np.float32)
    y = (xf * np.float32(inv_scale)).astype(np.float32)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    neg = np.signbit(flat)
    a = np.abs(flat.astype(np.float64))
    nan = np.isnan(flat)
    # index of the first representable magnitude >= a
    hi = np.searchsorted(_POS_VALUES, np.where(nan, 0.0, a), side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= 448.0, 0x7E, mag)
    code = mag.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    code = np.where(nan, 0x7F, code)
    out[:] = code
    return out.reshape(y.shape)


def widen_cache(arr: np.ndarray, fmt: str, scale: float = 1.0) -> np.ndarray:
    """Widen cache storage (float32 / bf16 bits / e4m3 codes) to float64.

    For E4M3 the stored value is code value x the tensor's float32 scale; a
    code value has at most 4 significant bits, so the float64 product is exact.
    """
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_to_f64(arr)
    if fmt == "fp8":
        return e4m3_to_f64(arr) * np.float64(np.float32(scale))
    raise ValueError(f"unknown cache format {fmt!r}")
