"""Seeded synthetic inputs shared by the GPU path's tests, the bench and the oracle checks.

This module only draws and quantises numbers. It holds none of the attention
arithmetic, so both sides of a parity test can take their inputs from it
without sharing any of the computation under test.

Recipe (the same for every workload):

* generator: ``numpy.random.default_rng(seed)`` (PCG64);
* draw order: q, k, v, dO, each ``standard_normal((B, T, H, hd))`` in float64;
* optional key outliers: per (b, h) in row-major order, ``round(frac * T)``
  distinct key rows from ``rng.choice(T, n, replace=False)`` drawn after dO,
  multiplied by 8 in float32 (a power of two, so exact);
* float32 storage: float64 -> float32 round-to-nearest-even;
* bfloat16 storage: the float32 values rounded to bfloat16 (round to nearest,
  ties to even), kept as their 16-bit patterns in ``uint16`` arrays;
* half storage: the float32 values rounded to IEEE binary16 (numpy's
  round-to-nearest-even conversion), kept as their 16-bit patterns.

All tensors are laid out [B, T, H, hd], row-major.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Case:
    """One attention problem: shapes, mask, scale and the stored inputs."""

    name: str
    B: int
    H: int
    T: int
    hd: int
    dtype: str
    causal: bool
    scale: float
    seed: int
    q: np.ndarray = field(repr=False)
    k: np.ndarray = field(repr=False)
    v: np.ndarray = field(repr=False)
    do: np.ndarray = field(repr=False)

    def f64(self, name: str) -> np.ndarray:
        """The exact values the device receives, widened to float64."""
        return _widen(getattr(self, name), self.dtype)

    def head_f64(self, name: str, b: int, h: int) -> np.ndarray:
        return _widen(getattr(self, name)[b, :, h, :], self.dtype)

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == F32 else 2


def _widen(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == F16:
        return np.ascontiguousarray(a).view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def make_case(name: str, B: int, H: int, T: int, hd: int, dtype: str, causal: bool, seed: int,
              scale: float | None = None, outlier_frac: float = 0.0) -> Case:
    rng = np.random.default_rng(seed)
    shape = (B, T, H, hd)
    arrs = [rng.standard_normal(shape).astype(np.float32) for _ in range(4)]
    q, k, v, do = arrs
    if outlier_frac > 0.0:
        n = int(round(outlier_frac * T))
        for b in range(B):
            for h in range(H):
                rows = rng.choice(T, n, replace=False)
                k[b, rows, h, :] *= np.float32(8.0)
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    if dtype == BF16:
        q, k, v, do = (f32_to_bf16_bits(a) for a in (q, k, v, do))
    elif dtype == F16:
        q, k, v, do = (a.astype(np.float16).view(np.uint16) for a in (q, k, v, do))
    elif dtype != F32:
        raise ValueError(dtype)
    return Case(name, B, H, T, hd, dtype, causal, float(scale), seed, q, k, v, do)


# The five workloads.  Names say what each is.
def tiny_case(causal: bool) -> Case:
    """One head, T=64, hd=16, float32, scale 1/sqrt(16), seed 0 (both masks)."""
    return make_case("tiny_T64_hd16_" + ("causal" if causal else "full"), 1, 1, 64, 16, F32, causal, 0, scale=0.25)


RAGGED_SHAPES = [(1, 4, 16, 8), (1, 4, 20, 8), (1, 2, 256, 32), (2, 2, 300, 64)]


def ragged_cases() -> list[Case]:
    """Causal float32 shapes with partial tiles; seeds 10..13 in listed order."""
    out = []
    for i, (B, H, T, hd) in enumerate(RAGGED_SHAPES):
        out.append(make_case(f"ragged_B{B}H{H}T{T}hd{hd}", B, H, T, hd, F32, True, 10 + i))
    return out


GPT2M = dict(B=64, H=16, T=1024, hd=64)


def gpt2m_case(dtype: str) -> Case:
    """GPT-2-medium-shaped causal attention (B64 H16 T1024 hd64), seed 2.

    The bfloat16 case uses the float32 case's draws rounded to bfloat16.
    """
    return make_case(f"gpt2m_{dtype}", GPT2M["B"], GPT2M["H"], GPT2M["T"], GPT2M["hd"], dtype, True, 2)


LONG = dict(B=4, H=16, T=8192, hd=128)


def long_case() -> Case:
    """Long-context causal attention (B4 H16 T8192 hd128), bfloat16, seed 4, 1% of key rows x8."""
    return make_case("long_bf16", LONG["B"], LONG["H"], LONG["T"], LONG["hd"], BF16, True, 4, outlier_frac=0.01)


# The lab of the fused-attention lesson: one head, no mask, float32, inputs
# uniform in [-2, 2) (the lesson's correctness inputs), scale 1/sqrt(d).
LAB_SIZES = (256, 512, 1024, 2048, 4096)
LAB_WIDTHS = (16, 64)


def lab_case(N: int, d: int, seed: int = 1) -> Case:
    """One head of N rows of width d: q, k, v uniform in [-2, 2) drawn in that order, float32."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.uniform(-2.0, 2.0, (1, N, 1, d)).astype(np.float32) for _ in range(3))
    do = np.zeros_like(q)
    return Case(f"lab_N{N}_d{d}", 1, 1, N, d, F32, False, 1.0 / math.sqrt(d), seed, q, k, v, do)
