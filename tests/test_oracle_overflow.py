"""Pins of the binary16 overflow analysis (oracle/overflow.py), CPU only.

Values printed by the "Lesson K23, fused attention" facts page, block
``overflow``: the threshold ln 65520 = 11.0901, and the probe row whose largest
score 10.3194 gives e^10.32 = 30320 in binary16, a naive sum of 30320 (the
other terms are absorbed), a safe sum of 1 and an overflow factor of 1.0747.
The page does not print the probe row's other scores; a row with the same max
and small other scores reproduces every printed number.
"""
import math

import numpy as np

from oracle import overflow


def test_threshold_is_ln_65520():
    assert round(overflow.THRESHOLD, 4) == 11.0901
    assert np.isfinite(np.float16(math.exp(overflow.THRESHOLD - 1e-6)))
    assert np.isinf(np.float16(math.exp(overflow.THRESHOLD + 1e-6)))
    assert float(np.finfo(np.float16).max) == overflow.F16_MAX


PROBE = [0.4, -1.3, 10.3194, 1.1, -0.2, 2.0, -3.5, 0.9]


def test_probe_row_numbers():
    assert float(np.float16(math.exp(10.3194))) == 30320.0
    p, total = overflow.naive_softmax_f16(PROBE)
    assert float(total) == 30320.0 and np.isfinite(p).all()
    ps, ts = overflow.safe_softmax_f16(PROBE)
    assert abs(float(ps.astype(np.float64).sum()) - 1.0) < 2e-3 and float(ps.max()) == float(np.float16(1.0 / float(ts)))
    f = overflow.overflow_factor(PROBE)
    assert round(f, 4) == 1.0747
    assert f == math.log(65520.0) / 10.3194 or abs(f - math.log(65520.0) / 10.3194) < 1e-9


def test_naive_overflows_safe_does_not():
    row = [12.0, 3.0, -1.0]
    p, total = overflow.naive_softmax_f16(row)
    assert np.isinf(total) and not np.isfinite(p).all()
    ps, ts = overflow.safe_softmax_f16(row)
    assert np.isfinite(ps).all() and np.isfinite(ts)
    ref = np.exp(np.array(row) - 12.0)
    ref /= ref.sum()
    assert np.abs(ps.astype(np.float64) - ref).max() < 1e-3


def test_overflow_factor_of_a_row_that_never_overflows():
    assert overflow.overflow_factor([0.0, 0.0, 0.0]) == math.inf
