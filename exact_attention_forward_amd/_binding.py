"""ctypes binding of the C ABI in include/fa.h: argument marshalling only.

Each ``fa_*`` function takes the same arguments as its C counterpart, in the
same order, and returns the C status code.  Pointer arguments accept a torch
tensor (its ``data_ptr()``), a plain integer address or None (NULL); the stream
accepts a ``torch.cuda.Stream``, an integer handle or None (default stream).
The shared library is loaded on first use; if it is missing the call raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

FA_F32 = 0
FA_BF16 = 1
FA_F16 = 2
FA_PREC_DEFAULT = 0
FA_PREC_BF16 = 1
FA_PREC_BF16X2 = 2

FA_OK = 0
FA_ERR_ARG = -1
FA_ERR_ALIGN = -2
FA_ERR_UNSUPPORTED = -3
FA_ERR_ALIAS = -4
FA_ERR_LAUNCH = -5
FA_ERR_TOO_LARGE = -6

# Every symbol include/fa.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "fa_forward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_backward_nows": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_backward_delta": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fa_backward_dq": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_backward_dkv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_backward_dq_delta": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_forward_splitkv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_forward_auto_splits": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "fa_forward_unfused": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_forward_norescale": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_forward_nomax": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_is_supported": (_I, [_I, _I]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
}

_LIB = None


class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"fa status {status}: {fa_status_string(status)}")
        self.status = status


def library_path() -> Path:
    return Path(__file__).resolve().parent / "libfa.so"


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        p = library_path()
        if not p.exists():
            raise RuntimeError(f"HIP library {p} is missing: build it with exact_attention_forward_amd.build.build()")
        L = ctypes.CDLL(str(p))
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def check(status: int) -> None:
    """Raise FaError for a non-zero status."""
    if status != FA_OK:
        raise FaError(status)


def fa_forward(q, k, v, o, lse, B, H, T, hd, scale, causal, dtype, prec, stream) -> int:
    return lib().fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, T, hd, scale, int(causal), dtype,
                            prec, _stream(stream))


def fa_forward_splitkv(q, k, v, o, lse, ws, B, H, T, hd, scale, causal, nsplit, dtype, prec, stream) -> int:
    return lib().fa_forward_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), B, H, T, hd, scale,
                                    int(causal), nsplit, dtype, prec, _stream(stream))


def fa_forward_auto_splits(B, H, T, hd, causal, dtype, prec) -> int:
    return lib().fa_forward_auto_splits(B, H, T, hd, int(causal), dtype, prec)


def fa_forward_unfused(q, k, v, o, scores, B, H, T, hd, scale, causal, dtype, stream) -> int:
    return lib().fa_forward_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(scores), B, H, T, hd, scale, int(causal),
                                    dtype, _stream(stream))


def fa_forward_norescale(q, k, v, o, lse, B, H, T, hd, scale, causal, dtype, stream) -> int:
    return lib().fa_forward_norescale(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, T, hd, scale, int(causal),
                                      dtype, _stream(stream))


def fa_forward_nomax(q, k, v, o, lse, B, H, T, hd, scale, causal, dtype, stream) -> int:
    return lib().fa_forward_nomax(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, T, hd, scale, int(causal), dtype,
                                  _stream(stream))


def fa_backward(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, hd, scale, causal, dtype, prec, stream) -> int:
    return lib().fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(delta), B, H, T, hd, scale, int(causal), dtype, prec, _stream(stream))


def fa_backward_nows(q, k, v, o, lse, dO, dq, dk, dv, B, H, T, hd, scale, causal, dtype, prec, stream) -> int:
    return lib().fa_backward_nows(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk),
                                  _ptr(dv), B, H, T, hd, scale, int(causal), dtype, prec, _stream(stream))


def fa_backward_delta(o, dO, delta, B, H, T, hd, dtype, stream) -> int:
    return lib().fa_backward_delta(_ptr(o), _ptr(dO), _ptr(delta), B, H, T, hd, dtype, _stream(stream))


def fa_backward_dq(q, k, v, lse, dO, delta, dq, B, H, T, hd, scale, causal, dtype, prec, stream) -> int:
    return lib().fa_backward_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(delta), _ptr(dq), B, H, T, hd,
                                scale, int(causal), dtype, prec, _stream(stream))


def fa_backward_dkv(q, k, v, lse, dO, delta, dk, dv, B, H, T, hd, scale, causal, dtype, prec, stream) -> int:
    return lib().fa_backward_dkv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(delta), _ptr(dk), _ptr(dv), B,
                                 H, T, hd, scale, int(causal), dtype, prec, _stream(stream))


def fa_backward_dq_delta(q, k, v, o, lse, dO, dq, delta, B, H, T, hd, scale, causal, dtype, prec, stream) -> int:
    return lib().fa_backward_dq_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(delta), B,
                                      H, T, hd, scale, int(causal), dtype, prec, _stream(stream))


def fa_is_supported(hd, dtype) -> int:
    return lib().fa_is_supported(hd, dtype)


def fa_status_string(status) -> str:
    return lib().fa_status_string(status).decode()
