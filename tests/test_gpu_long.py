"""Long sequences (T up to 65536, few heads) through the C ABI, checked on sampled rows and key columns.

The full-head oracle does not fit these lengths, but the definition decomposes by query row.  Under the
causal mask row i sees keys 0..i only, so its O, L and dQ are those of the single-query problem (query i,
keys and values 0..i, no mask).  The loss is a sum over rows, so the dK and dV of key j are the sums, over
the rows i >= j, of each single-query problem's dK and dV at j: for the last keys only the last rows
contribute.  Each piece is one call of the oracle; the checks use the same tolerances as every other
parity test (float32: 2e-5, with 1e-3 for dV at T >= 4096; 16-bit inputs: 2e-2).
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I
from oracle import attention as oracle

from gpu_util import BF16_TOL, F32_TOL, run_case, to_device

pytestmark = pytest.mark.gpu

LAST_KEYS = 48

# (B, H, T, hd, dtype, precision, seed)
LONG = [(1, 2, 65536, 64, I.BF16, fa.FA_PREC_BF16, 31),
        (1, 1, 32768, 128, I.BF16, fa.FA_PREC_BF16X2, 32),
        (1, 1, 16384, 64, I.F32, fa.FA_PREC_DEFAULT, 33)]


def _single_query(q, k, v, do, i, scale):
    """Oracle forward and backward of query row i against keys 0..i (what causal row i computes)."""
    O, L, _ = oracle.head_forward(q[i:i + 1], k[:i + 1], v[:i + 1], scale, False)
    dq, dk, dv, _ = oracle.head_backward(q[i:i + 1], k[:i + 1], v[:i + 1], do[i:i + 1], scale, False)
    return O[0], L[0], dq[0], dk, dv


@pytest.mark.parametrize("B,H,T,hd,dtype,prec,seed", LONG,
                         ids=[f"T{t[2]}_hd{t[3]}_{t[4]}" for t in LONG])
def test_long_sequence_sampled(B, H, T, hd, dtype, prec, seed):
    c = I.make_case(f"long_T{T}_hd{hd}", B, H, T, hd, dtype, True, seed)
    print(f"[long] B{B} H{H} T{T} hd{hd} {dtype} prec={prec}", flush=True)
    out = run_case(c, prec)
    host = {n: out[n].cpu().numpy().astype(np.float64) for n in ("O", "L", "dQ", "dK", "dV")}
    rows = [0, 1, 4095, T // 2 + 17, T - 1]
    k0 = T - LAST_KEYS
    worst = {}

    def note(name, got, ref):
        worst[name] = max(worst.get(name, 0.0), float(np.abs(got - ref).max()))

    for h in range(H):
        q, k, v, do = (c.head_f64(n, 0, h) for n in ("q", "k", "v", "do"))
        for i in rows:
            O, L, dq, _, _ = _single_query(q, k, v, do, i, c.scale)
            note("O", host["O"][0, i, h], O)
            note("L", host["L"][0, h, i], L)
            note("dQ", host["dQ"][0, i, h], dq)
        dK = np.zeros((LAST_KEYS, hd))
        dV = np.zeros((LAST_KEYS, hd))
        for i in range(k0, T):
            _, _, _, dk, dv = _single_query(q, k, v, do, i, c.scale)
            dK[:i + 1 - k0] += dk[k0:]
            dV[:i + 1 - k0] += dv[k0:]
        note("dK", host["dK"][0, k0:, h], dK)
        note("dV", host["dV"][0, k0:, h], dV)
    print(f"[long] T{T} hd{hd} {dtype}: {worst}", flush=True)
    if dtype == I.F32:
        tol = {n: F32_TOL for n in worst}
        tol["dV"] = 1e-3  # float32 dV at T >= 4096
    else:
        tol = {n: BF16_TOL for n in worst}
    bad = {n: e for n, e in worst.items() if not e <= tol[n]}
    assert not bad, f"errors over tolerance: {bad} (all: {worst})"


@pytest.mark.parametrize("nsplit", [5, 16])
def test_long_sequence_split_forward_sampled(nsplit):
    """The split-key forward at T = 65536 (partial outputs of 8.4M floats each in the workspace)."""
    B, H, T, hd = 1, 2, 65536, 64
    c = I.make_case(f"long_split_T{T}", B, H, T, hd, I.BF16, True, 34)
    print(f"[long split] B{B} H{H} T{T} hd{hd} bf16 nsplit={nsplit}", flush=True)
    q, k, v = (to_device(c, n) for n in ("q", "k", "v"))
    o = torch.full((B, T, H, hd), float("nan"), device="cuda")
    lse = torch.full((B, H, T), float("nan"), device="cuda")
    ws = torch.full((nsplit * (B * T * H * hd + B * H * T),), float("nan"), device="cuda")
    fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, ws, B, H, T, hd, c.scale, 1, nsplit, fa.FA_BF16,
                                   fa.FA_PREC_BF16, None))
    torch.cuda.synchronize()
    O_g, L_g = o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(O_g).all() and np.isfinite(L_g).all()
    worst = {}
    for h in range(H):
        q_, k_, v_ = (c.head_f64(n, 0, h) for n in ("q", "k", "v"))
        for i in [0, 13107, 32768, T - 2, T - 1]:
            O, L, _ = oracle.head_forward(q_[i:i + 1], k_[:i + 1], v_[:i + 1], c.scale, False)
            worst["O"] = max(worst.get("O", 0.0), float(np.abs(O_g[0, i, h] - O[0]).max()))
            worst["L"] = max(worst.get("L", 0.0), float(abs(L_g[0, h, i] - L[0])))
    print(f"[long split] nsplit={nsplit}: {worst}", flush=True)
    assert all(e <= BF16_TOL for e in worst.values()), worst
