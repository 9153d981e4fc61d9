"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Tolerance per element, from the bound stated for this path:
    |gpu - ref| <= 2 * ulp16(|ref|) + 1e-3 * sqrt(K)
where ref is the oracle's fp16 result, ulp16(x) = 2^(floor(log2 x) - 10) for
x >= 2^-14 (the spacing of fp16 values in x's binade) and 2^-24 below.
Infinities must match exactly (sign included) and NaN must meet NaN.
"""
from __future__ import annotations

import math

import numpy as np


def ulp16(x: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(a.shape, 2.0 ** -24)
    big = a >= 2.0 ** -14
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(big, a, 1.0)))
    out[big] = np.exp2(e[big] - 10.0)
    return out


def tolerance(ref: np.ndarray, K: int) -> np.ndarray:
    return 2.0 * ulp16(ref) + 1e-3 * math.sqrt(max(K, 0))


def as_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits)
    if b.dtype == np.float16:
        return b.astype(np.float64)
    return b.astype(np.uint16).view(np.float16).astype(np.float64)


def compare(gpu_bits: np.ndarray, ref_bits: np.ndarray, K: int):
    """(ok, worst_ratio, n_bad, first_bad_index) for elementwise parity."""
    g = as_f64(gpu_bits)
    r = as_f64(ref_bits)
    assert g.shape == r.shape, (g.shape, r.shape)
    nan_r, nan_g = np.isnan(r), np.isnan(g)
    inf_r = np.isinf(r)
    bad = (nan_r != nan_g)
    bad |= inf_r & ~(g == r)
    fin = ~nan_r & ~inf_r
    tol = tolerance(r, K)
    err = np.zeros_like(r)
    err[fin] = np.abs(g[fin] - r[fin])
    bad |= fin & ~(err <= tol)          # NaN/inf on the GPU side fails here too
    ratio = np.where(fin, err / tol, 0.0)
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    idx = np.argwhere(bad)
    return (not bad.any()), worst, int(bad.sum()), (tuple(idx[0]) if idx.size else None)


def assert_parity(gpu_bits, ref_bits, K: int, what: str = ""):
    ok, worst, nbad, first = compare(gpu_bits, ref_bits, K)
    if not ok:
        g = as_f64(gpu_bits)[first]
        r = as_f64(ref_bits)[first]
        raise AssertionError(f"{what}: {nbad} elements out of tolerance; first at {first}: "
                             f"gpu={g!r} ref={r!r} tol={float(tolerance(np.array([r]), K)[0])!r}; "
                             f"worst err/tol={worst:.3f}")
    return worst
