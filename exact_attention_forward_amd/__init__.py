"""Exact attention (online-softmax forward, recomputing backward) for AMD MI355X.

The computation lives in the HIP library ``libfa.so`` (C ABI: include/fa.h),
built from ``csrc/`` by ``exact_attention_forward_amd.build``.  This package
holds the ctypes binding (``fa_*``, same names and arguments as the C entry
points), a torch convenience layer (``forward``, ``backward`` and the autograd
operation ``attention``; torch only provides memory and streams) and the seeded
input generators (``inputs``).
"""
from ._binding import (FA_BF16, FA_F16, FA_ERR_ALIAS, FA_ERR_ALIGN, FA_ERR_ARG, FA_ERR_LAUNCH, FA_ERR_TOO_LARGE, FA_ERR_UNSUPPORTED, FA_F32,
                       FA_OK, FA_PREC_BF16, FA_PREC_BF16X2, FA_PREC_DEFAULT, FaError, check, fa_backward,
                       fa_backward_delta, fa_backward_dkv, fa_backward_nows, fa_backward_dq, fa_backward_dq_delta, fa_forward,
                       fa_forward_auto_splits, fa_forward_nomax, fa_forward_norescale, fa_forward_splitkv, fa_forward_unfused, fa_is_supported, fa_status_string, lib, library_path)


def __getattr__(name):
    if name in ("forward", "backward", "attention"):
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
