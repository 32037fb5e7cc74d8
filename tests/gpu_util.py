"""Helpers shared by the GPU tests: device copies of seeded cases and oracle comparison."""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I
from oracle import attention as oracle

F32_TOL = 2e-5
BF16_TOL = 2e-2


def to_device(case: I.Case, name: str) -> torch.Tensor:
    a = getattr(case, name)
    if case.dtype == I.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if case.dtype == I.F16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_case(case: I.Case, prec: int = fa.FA_PREC_DEFAULT, poison: bool = True, stream=None):
    """Forward + backward through the C ABI.  Outputs start as NaN so unwritten elements show."""
    q, k, v, do = (to_device(case, n) for n in ("q", "k", "v", "do"))
    B, T, H, hd = q.shape
    dtc = {I.BF16: fa.FA_BF16, I.F16: fa.FA_F16}.get(case.dtype, fa.FA_F32)
    fill = float("nan") if poison else 0.0
    mk = lambda *s: torch.full(s, fill, device="cuda", dtype=torch.float32)
    o, lse = mk(B, T, H, hd), mk(B, H, T)
    dq, dk, dv, delta = mk(B, T, H, hd), mk(B, T, H, hd), mk(B, T, H, hd), mk(B, H, T)
    fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, case.scale, case.causal, dtc, prec, stream))
    fa.check(fa.fa_backward(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, T, hd, case.scale, case.causal, dtc, prec,
                            stream))
    torch.cuda.synchronize()
    return dict(O=o, L=lse, dQ=dq, dK=dk, dV=dv, D=delta)


def oracle_head(case: I.Case, b: int, h: int):
    q, k, v, do = (case.head_f64(n, b, h) for n in ("q", "k", "v", "do"))
    O, L, _ = oracle.head_forward(q, k, v, case.scale, case.causal)
    dQ, dK, dV, D = oracle.head_backward(q, k, v, do, case.scale, case.causal)
    return dict(O=O, L=L, dQ=dQ, dK=dK, dV=dV, D=D)


def head_errors(case: I.Case, out: dict, b: int, h: int) -> dict:
    ref = oracle_head(case, b, h)
    err = {}
    for n in ("O", "L", "dQ", "dK", "dV", "D"):
        g = out[n][b, h].cpu().numpy() if n in ("L", "D") else out[n][b, :, h].cpu().numpy()
        err[n] = float(np.abs(g.astype(np.float64) - ref[n]).max())
    return err


def heads_errors(case: I.Case, out: dict, heads) -> dict:
    """Max abs error over the given (b, h) heads, with each output copied to the host once."""
    host = {n: t.cpu().numpy() for n, t in out.items()}
    worst = {}
    for b, h in heads:
        ref = oracle_head(case, b, h)
        for n in ("O", "L", "dQ", "dK", "dV", "D"):
            g = host[n][b, h] if n in ("L", "D") else host[n][b, :, h]
            worst[n] = max(worst.get(n, 0.0), float(np.abs(g.astype(np.float64) - ref[n]).max()))
    return worst


def full_errors(case: I.Case, out: dict) -> dict:
    """Max abs error over every head (for small cases)."""
    worst = {}
    for b in range(case.B):
        for h in range(case.H):
            for n, e in head_errors(case, out, b, h).items():
                worst[n] = max(worst.get(n, 0.0), e)
    return worst


def assert_within(err: dict, tol: float, what: str, names=("O", "L", "dQ", "dK", "dV")):
    bad = {n: err[n] for n in names if not err[n] <= tol}
    assert not bad, f"{what}: errors over {tol}: {bad} (all: {err})"
