"""Torch-tensor convenience layer over the C ABI.

torch supplies device memory and the current stream; every step of the
computation runs in the HIP library.  Inputs are contiguous [B, T, H, hd]
device tensors of one dtype (float32, bfloat16 or float16) on one device;
outputs are float32.  Every tensor argument is checked here, before the
library is called: the C ABI sees only raw pointers and would read a tensor
of another dtype or size out of bounds.  ``attention`` wraps the two calls
as one autograd operation.
"""
from __future__ import annotations

import math

import torch

from . import _binding as _b
from ._binding import FA_BF16, FA_F16, FA_F32, FA_PREC_DEFAULT, check


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _on_device(t: torch.Tensor) -> bool:
    """True for a GPU tensor (the library takes device pointers only)."""
    return bool(t.is_cuda)


def _inputs(q: torch.Tensor, *others: torch.Tensor):
    """[B, T, H, hd] inputs: one shape, one dtype, one device, contiguous, on the GPU."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("expected [B, T, H, hd] tensors")
    _dtype_code(q)
    for t in (q, *others):
        if not isinstance(t, torch.Tensor):
            raise TypeError("inputs must be torch tensors")
        if t.dtype != q.dtype:
            raise TypeError(f"inputs must share one dtype: {t.dtype} vs {q.dtype}")
        if t.shape != q.shape:
            raise ValueError(f"inputs must share one shape: {tuple(t.shape)} vs {tuple(q.shape)}")
        if not _on_device(t) or t.device != q.device:
            raise ValueError("inputs must be device tensors on one device")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    B, T, H, hd = q.shape
    return B, T, H, hd


def _f32(t, shape, device, name: str) -> None:
    """A float32 tensor of the given shape, contiguous, on `device`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not _on_device(t) or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return torch.cuda.current_stream(device)


def forward(q, k, v, scale: float | None = None, causal: bool = True, prec: int = FA_PREC_DEFAULT, stream=None):
    """Returns (o [B, T, H, hd] float32, lse [B, H, T] float32)."""
    B, T, H, hd = _inputs(q, k, v)
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    o = torch.empty((B, T, H, hd), device=q.device, dtype=torch.float32)
    lse = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    stream = _stream(q.device) if stream is None else stream
    check(_b.fa_forward(q, k, v, o, lse, B, H, T, hd, scale, causal, _dtype_code(q), prec, stream))
    return o, lse


def backward(q, k, v, o, lse, do, scale: float | None = None, causal: bool = True, prec: int = FA_PREC_DEFAULT,
             stream=None):
    """Returns (dq, dk, dv [B, T, H, hd] float32, delta [B, H, T] float32).

    o and lse are the forward's outputs: float32 [B, T, H, hd] and [B, H, T].
    """
    B, T, H, hd = _inputs(q, k, v, do)
    _f32(o, (B, T, H, hd), q.device, "o")
    _f32(lse, (B, H, T), q.device, "lse")
    scale = 1.0 / math.sqrt(hd) if scale is None else scale
    dq = torch.empty((B, T, H, hd), device=q.device, dtype=torch.float32)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    delta = torch.empty((B, H, T), device=q.device, dtype=torch.float32)
    stream = _stream(q.device) if stream is None else stream
    check(_b.fa_backward(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, T, hd, scale, causal, _dtype_code(q), prec,
                         stream))
    return dq, dk, dv, delta


class _Attention(torch.autograd.Function):
    """fa_forward in the forward pass, fa_backward in the backward pass (O and L saved between)."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, prec):
        o, lse = forward(q, k, v, scale, causal, prec)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (scale, causal, prec)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, prec = ctx.cfg
        # the library takes dO in the inputs' dtype
        do = do.to(q.dtype).contiguous()
        dq, dk, dv, _ = backward(q, k, v, o, lse, do, scale, causal, prec)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None


def attention(q, k, v, scale: float | None = None, causal: bool = True, prec: int = FA_PREC_DEFAULT):
    """O = softmax(mask(scale q k^T)) v as an autograd operation: returns o (float32 [B, T, H, hd]);
    o.backward(dO) runs fa_backward with dO rounded to the inputs' dtype and leaves dq, dk, dv in
    q.grad, k.grad, v.grad, rounded to the inputs' dtype."""
    return _Attention.apply(q, k, v, scale, causal, prec)
