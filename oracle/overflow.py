"""Overflow of the softmax without the max subtracted, in IEEE binary16.

Test infrastructure (see the package docstring).

The "Lesson K23, fused attention" facts page (block ``overflow``): in binary16
the largest finite number is 65504, and e^s rounds to infinity once
e^s >= 65520 (halfway to 2^16, where round-to-nearest-even goes up), i.e. once
s >= ln 65520 = 11.0901.  Its "naive" softmax rounds the exponential, the
running sum and the division each to binary16 without subtracting the row
max; the "safe" one subtracts the max first, so the largest exponential is 1.
The overflow factor of a row is the smallest factor by which its scores could
be scaled before the naive binary16 sum overflows.
"""
from __future__ import annotations

import math

import numpy as np

F16_MAX = 65504.0
THRESHOLD = math.log(65520.0)


def _exp16(x: float) -> np.float16:
    with np.errstate(over="ignore"):
        return np.float16(math.exp(float(x)) if x < 700 else math.inf)


def naive_sum_f16(s) -> np.float16:
    """sum_j fl16(e^{s_j}), accumulated left to right in binary16."""
    acc = np.float16(0.0)
    with np.errstate(over="ignore"):
        for x in s:
            acc = np.float16(np.float32(acc) + np.float32(_exp16(x)))
    return acc


def naive_softmax_f16(s):
    """Weights fl16(fl16(e^{s_j}) / sum), no max subtracted."""
    total = naive_sum_f16(s)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        return np.array([np.float16(np.float32(_exp16(x)) / np.float32(total)) for x in s], np.float16), total


def safe_softmax_f16(s):
    """The same with the row max subtracted before the exponential."""
    m = max(float(x) for x in s)
    return naive_softmax_f16([float(x) - m for x in s])


def overflow_factor(s, hi: float = 64.0, iters: int = 200) -> float:
    """Smallest f >= 0 with naive_sum_f16(f * s) not finite (bisection), inf if none below `hi`."""
    s = [float(x) for x in s]
    if np.isfinite(naive_sum_f16([hi * x for x in s])):
        return math.inf
    lo = 0.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if np.isfinite(naive_sum_f16([mid * x for x in s])):
            lo = mid
        else:
            hi = mid
    return hi
