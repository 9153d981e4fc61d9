"""Seeded synthetic operands for the fp16 NT GEMM.

This module is the only code shared by the HIP path's tests/bench and the
CPU oracle's checks.  It produces fp16 matrices from a seed and holds none
of the GEMM's arithmetic.

Generator (counter-based, so any element can be produced independently):

* SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014; constants as in Vigna's
  public-domain ``splitmix64.c``) applied to the counter
  ``x = seed*0x9E3779B97F4A7C15 + stream*0xD1B54A32D192ED03 + idx``
  (mod 2^64), where ``stream`` is 0 for A and 1 for B and ``idx`` is the
  row-major element index.
* ``u = (z >> 11) * 2^-53`` is uniform on [0, 1).
* uniform[lo, hi]: ``lo + (hi - lo) * u`` in fp64.
* normal(0, sigma): Box-Muller on the pair (u[2i], u[2i+1]) with
  r = sqrt(-2 ln(1 - u[2i])), t = 2 pi u[2i+1]: element 2i gets
  ``sigma * r cos t`` and element 2i+1 ``sigma * r sin t``; then clipped.
* the fp64 value is rounded to fp16 by numpy (round-to-nearest-even).

Large matrices are produced in chunks so that the temporaries stay small.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_STREAM = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_A = 0
STREAM_B = 1
_CHUNK = 1 << 22


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output for state ``x`` (uint64 array), i.e. the value the
    generator returns after advancing its state to ``x + golden``."""
    with np.errstate(over="ignore"):
        z = x + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """u in [0, 1) for element indices start .. start+count-1."""
    with np.errstate(over="ignore"):
        base = (np.uint64(seed) * _GOLDEN + np.uint64(stream) * _STREAM)
        idx = np.arange(start, start + count, dtype=np.uint64)
        z = splitmix64(base + idx)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _uniform_values(dist: dict, seed: int, stream: int, start: int, count: int) -> np.ndarray:
    lo, hi = float(dist["lo"]), float(dist["hi"])
    return lo + (hi - lo) * uniform01(seed, stream, start, count)


def _normal_values(dist: dict, seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Box-Muller gives one normal per element: element 2i uses the cosine
    of the pair (u[2i], u[2i+1]) and element 2i+1 the sine of the same pair
    (the standard two-output form), so every element is N(0, 1)."""
    if start % 2:
        raise ValueError("normal chunks must start on an even index")
    n2 = count + (count % 2)
    u = uniform01(seed, stream, start, n2).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
    theta = 2.0 * np.pi * u[:, 1]
    z = np.empty(n2, dtype=np.float64)
    z[0::2] = r * np.cos(theta)
    z[1::2] = r * np.sin(theta)
    z = z[:count] * float(dist["sigma"])
    clip = float(dist.get("clip", np.inf))
    return np.clip(z, -clip, clip)


def generate(rows: int, cols: int, seed: int, stream: int, dist: dict) -> np.ndarray:
    """rows x cols fp16 matrix (numpy float16, row-major)."""
    n = int(rows) * int(cols)
    out = np.empty(n, dtype=np.float16)
    for s in range(0, n, _CHUNK):
        c = min(_CHUNK, n - s)
        if dist["kind"] == "normal":
            v = _normal_values(dist, seed, stream, s, c)
        elif dist["kind"] == "uniform":
            v = _uniform_values(dist, seed, stream, s, c)
        else:
            raise ValueError(f"unknown distribution {dist['kind']!r}")
        out[s:s + c] = v.astype(np.float16)
    return out.reshape(rows, cols)


def operands(M: int, N: int, K: int, seed: int, dist: dict):
    """(A, B): A is M x K, B is N x K, both fp16 numpy arrays."""
    return (generate(M, K, seed, STREAM_A, dist),
            generate(N, K, seed, STREAM_B, dist))


def batched_operands(batch: int, M: int, N: int, K: int, seed: int, dist: dict):
    """(A, B) of `batch` products: A is batch x M x K, B is batch x N x K,
    drawn as one (batch*M) x K and one (batch*N) x K matrix and split into
    batch entries in order."""
    A, B = operands(batch * M, batch * N, K, seed, dist)
    return A.reshape(batch, M, K), B.reshape(batch, N, K)


def periodic_index(rows: int, period: int, shift: int = 0) -> np.ndarray:
    """Row r of an operand built from a small seeded pattern matrix P of
    `period` rows is P[(r + shift) % period]; this returns those pattern
    indices (int64).  Operands of several GiB are built this way on the
    device from a P that is cheap to draw, and the same indices give the
    host-side rows of any sample."""
    return (np.arange(rows, dtype=np.int64) + int(shift)) % int(period)
