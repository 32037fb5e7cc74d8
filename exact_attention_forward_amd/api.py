"""Torch-tensor convenience layer over the C ABI.

torch supplies device memory and the current stream; every step of the
computation runs in the HIP library.  Inputs are contiguous [B, T, H, hd]
device tensors of dtype float32, bfloat16 or float16; outputs are float32.
"""
from __future__ import annotations

import math

import torch

from ._binding import (FA_BF16, FA_F16, FA_F32, FA_PREC_DEFAULT, check, fa_backward, fa_backward_delta, fa_backward_dkv,
                       fa_backward_dq, fa_forward)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _shape(q: torch.Tensor, *others: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected [B, T, H, hd] tensors")
    for t in (q, *others):
        if t.shape != q.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("inputs must be contiguous device tensors of one shape")
    B, T, H, hd = q.shape
    return B, T, H, hd


def forward(q, k, v, scale: float | None = None, causal: bool = True, prec: int = FA_PREC_DEFAULT, stream=None):
    """Returns (o [B, T, H, hd] float32, lse [B, H, T] float32)."""
    B, T, H, hd = _shape(q, k, v)
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    o = torch.empty((B, T, H, hd), device=q.device, dtype=torch.float32)
    lse = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    check(fa_forward(q, k, v, o, lse, B, H, T, hd, scale, causal, _dtype_code(q), prec, stream))
    return o, lse


def backward(q, k, v, o, lse, do, scale: float | None = None, causal: bool = True, prec: int = FA_PREC_DEFAULT,
             stream=None):
    """Returns (dq, dk, dv [B, T, H, hd] float32, delta [B, H, T] float32)."""
    B, T, H, hd = _shape(q, k, v, do)
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    dq = torch.empty((B, T, H, hd), device=q.device, dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    delta = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    check(fa_backward(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, T, hd, scale, causal, _dtype_code(q), prec,
                      stream))
    return dq, dk, dv, delta
