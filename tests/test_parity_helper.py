"""The tolerance rule itself (CPU)."""
import math

import numpy as np

from tests.parity import compare, tolerance, ulp16


def test_ulp16_binades():
    xs = np.array([1.0, 1.5, 2.0, 1000.0, 2048.0, 65504.0, 2.0 ** -14, 2.0 ** -20, 0.0])
    want = [2.0 ** -10, 2.0 ** -10, 2.0 ** -9, 0.5, 2.0, 32.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24]
    assert list(ulp16(xs)) == want


def test_tolerance_values():
    assert math.isclose(float(tolerance(np.array([0.0]), 64)[0]), 2 * 2.0 ** -24 + 0.008)
    assert math.isclose(float(tolerance(np.array([1.0]), 4096)[0]), 2 * 2.0 ** -10 + 0.064)


def test_compare_flags():
    r = np.array([1.0, np.inf, np.nan, 2.0], dtype=np.float16)
    assert compare(r.copy(), r, 64)[0]
    g = r.copy(); g[1] = 65504
    assert not compare(g, r, 64)[0]
    g = r.copy(); g[2] = 0
    assert not compare(g, r, 64)[0]
    g = r.copy(); g[3] = np.nan
    assert not compare(g, r, 64)[0]
    # K = 1: tol(1.0) = 2^-9 + 0.001 ~ 0.00295
    g = r.copy(); g[0] = 1.0 + 2.0 ** -10          # 0.00098 off: inside
    assert compare(g, r, 1)[0]
    g = r.copy(); g[0] = 1.0 + 4 * 2.0 ** -10      # 0.0039 off: outside
    assert not compare(g, r, 1)[0]
