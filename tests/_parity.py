"""Comparison of GPU decode outputs with the oracle's, shared by the GPU tests.

Every check compares all output rows.  Three things are checked, and the
figures are written as one JSON line per check to the file named by the
environment variable PA_PARITY_LOG (when it is set):

1. The stated tolerance: max |gpu - oracle| <= 1e-5 (fp32 cache), 2e-2
   (bf16), 6e-2 (fp8-e4m3), no NaN or Inf.

2. For bf16 outputs, the error split into its two sources.  ``rounding`` is
   |RNE_bf16(oracle) - oracle|, what rounding the exact result once to bf16
   costs; ``kernel`` is |gpu - RNE_bf16(oracle)|, counted in bf16 ulps of the
   rounded oracle value.

3. For bf16 outputs of decode (one query per row), a bound derived from the
   kernel's arithmetic, element by element:

       |gpu - o| <= ulp(gpu) / 2 + 2 eps / (1 - eps) * S + 2 (n + 32) 2^-24 M

   o is the oracle's exact output, S = max_t |V_t[d] - o[d]| and
   M = max_t |V_t[d]| over the row's visible positions t, n = ceil(L / 16).
   The terms: the one final rounding to bf16; the exponentials rounded to bf16
   before the P.V product (relative error <= 2^-9 per weight, plus 2^-12 for
   the float32 logits and exp2), which perturbs the normalised weights w_t to
   w_t (1 + e_t) / (1 + sum_u w_u e_u) and so moves the output by
   sum_t w_t (e_t - e_mean) (V_t - o) / (1 + e_mean), at most 2 eps S / (1 - eps);
   float32 accumulation of the sums over n tiles and the merges of pieces.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
EPS_W = 2.0 ** -9 + 2.0 ** -12        # per-weight relative error of the kernel's P


def round_bf16(x):
    """float64 -> the nearest bfloat16 value (ties to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)          # exponent of one bf16 ulp (subnormals: 2^-133)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def ulp_bf16(v):
    """One bf16 ulp at the bf16 value v: 2^(e - 8) for |v| in [2^(e-1), 2^e)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    return np.ldexp(1.0, np.maximum(np.where(v == 0, -200, e - 8), -133))


def _log(rec):
    path = os.environ.get("PA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def value_stats(q, q_fmt, k_cache, v_cache, fmt, block_tables, context_lens, ref,
                k_scale=1.0, v_scale=1.0):
    """Per (sequence, query head, dim): S = max_t |V_t - o| and M = max_t |V_t|
    over the sequence's positions, and per sequence n = ceil(L / 16)."""
    B, Hq, D = ref.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    S = np.zeros((B, Hq, D))
    M = np.zeros((B, Hq, D))
    n = np.zeros(B)
    for s in range(B):
        L = int(context_lens[s])
        n[s] = -(-L // 16)
        if L == 0:
            continue
        for g in range(Hkv):
            V = oracle.widen_cache(oracle.gather_kv(v_cache, block_tables[s], L, g), fmt, v_scale)
            vm = np.abs(V).max(axis=0)
            for h in range(g * G, (g + 1) * G):
                S[s, h] = np.abs(V - ref[s, h]).max(axis=0)
                M[s, h] = vm
    return S, M, n


def check(got, ref, fmt, label, out_bf16=True, stats=None):
    """Compares every element of ``got`` (float64 values of the GPU output)
    with ``ref`` (the oracle's float64 output) as described in the module
    docstring.  ``stats`` = value_stats(...) enables the derived bound (decode
    rows, [B, Hq, D]).  Returns the record that was logged."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert np.all(np.isfinite(ref)), f"{label}: oracle rows missing"
    err = np.abs(got - ref)
    rec = {"check": label, "fmt": fmt, "elements": int(got.size),
           "max_abs_err": float(err.max()) if err.size else 0.0, "tol": TOL[fmt]}
    if out_bf16 and got.size:
        r = round_bf16(ref)
        ulps = np.abs(got - r) / ulp_bf16(r)
        rec.update({
            "rounding_max": float(np.abs(r - ref).max()),
            "kernel_max": float(np.abs(got - r).max()),
            "exact_frac": float(np.mean(got == r)),
            "within_1ulp_frac": float(np.mean(ulps <= 1.0)),
            "max_ulps": float(ulps.max()),
        })
        if stats is not None:
            S, M, n = stats
            bound = (0.5 * ulp_bf16(np.abs(got)) + 2 * EPS_W / (1 - EPS_W) * S +
                     2 * (n[:, None, None] + 32) * 2.0 ** -24 * M)
            rec["max_err_over_bound"] = float((err / bound).max())
    _log(rec)
    print(f"  {label}: {json.dumps(rec)}", flush=True)
    assert rec["max_abs_err"] <= TOL[fmt], f"{label}: max abs error {rec['max_abs_err']} > {TOL[fmt]}"
    if "max_err_over_bound" in rec:
        assert rec["max_err_over_bound"] <= 1.0, f"{label}: error above the derived bound"
    return rec


def check_mean_rows(got, ref, lens, M, label):
    """q = 0: every weight is 1 / L and the output is the mean of the V rows.
    The kernel's weights are then exactly 1 and its sums are float32 sums of
    the V rows, so each element is RNE_bf16(mean) unless float32 rounding moved
    the sum across a rounding midpoint: at most 1 ulp, or the float32 bound
    (n + 32) 2^-24 M when the mean is tiny.  A row in which one position was
    read from the wrong place is off by about |V_wrong - V_right| / L, several
    ulps of the mean in most of its elements, so every row must also be exact
    in at least 90% of its elements."""
    got = np.asarray(got, dtype=np.float64)
    r = round_bf16(ref)
    ulps = np.abs(got - r) / ulp_bf16(r)
    n = -(-np.asarray(lens, dtype=np.int64) // 16)
    slack = (n[:, None, None] + 32) * 2.0 ** -24 * M
    ok = (ulps <= 1.0) | (np.abs(got - ref) <= slack)
    exact_row = np.mean(got == r, axis=-1)
    rec = {"check": label, "fmt": "bf16", "elements": int(got.size),
           "exact_frac": float(np.mean(got == r)), "max_ulps": float(ulps.max()),
           "min_row_exact_frac": float(exact_row.min()),
           "max_abs_err": float(np.abs(got - ref).max())}
    _log(rec)
    print(f"  {label}: {json.dumps(rec)}", flush=True)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert ok.all(), f"{label}: {int((~ok).sum())} elements more than 1 ulp from the mean"
    assert exact_row.min() >= 0.9, f"{label}: a row is exact in only {exact_row.min():.2f}"
    return rec
