"""The lab of the fused-attention lesson on the GPU, through the C ABI.

For each size N in {256, ..., 4096} and width d in {16, 64} (one head, no
mask, float32, inputs uniform in [-2, 2) with seed 1), the fused forward
(fa_forward), the unfused three-kernel forward (fa_forward_unfused) and the
no-rescale control (fa_forward_norescale) are checked element by element
against the float64 reference with the lesson's error bound (oracle/checker.py),
on the rows the lab checks (all up to N = 1024, the first 64 above).  The fused
and unfused kernels must pass; the control must fail (its key blocks are 32
keys, so every lab size raises some row's max after its first block), and must
pass when a single key block covers the whole sequence.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I
from oracle import checker

pytestmark = pytest.mark.gpu


def run_kinds(c):
    q, k, v = (torch.from_numpy(getattr(c, n)).cuda() for n in ("q", "k", "v"))
    N, d = c.T, c.hd
    out = {}
    for kind in ("fused", "unfused", "broken"):
        o = torch.full((1, N, 1, d), float("nan"), device="cuda")
        lse = torch.full((1, 1, N), float("nan"), device="cuda")
        if kind == "fused":
            fa.check(fa.fa_forward(q, k, v, o, lse, 1, 1, N, d, c.scale, 0, fa.FA_F32, 0, None))
        elif kind == "unfused":
            s = torch.empty((1, 1, N, N), device="cuda")
            fa.check(fa.fa_forward_unfused(q, k, v, o, s, 1, 1, N, d, c.scale, 0, fa.FA_F32, None))
        else:
            fa.check(fa.fa_forward_norescale(q, k, v, o, lse, 1, 1, N, d, c.scale, 0, fa.FA_F32, None))
        torch.cuda.synchronize()
        out[kind] = o[0, :, 0, :].cpu().numpy()
    return out


@pytest.mark.parametrize("d", I.LAB_WIDTHS)
@pytest.mark.parametrize("N", I.LAB_SIZES)
def test_lab_checker(N, d):
    c = I.lab_case(N, d)
    rows = checker.rows_checked(N)
    ref, bound = checker.reference_and_bound(c.q[0, :, 0, :], c.k[0, :, 0, :], c.v[0, :, 0, :], c.scale, rows)
    out = run_kinds(c)
    res = {kind: checker.check(o[rows], ref, bound) for kind, o in out.items()}
    print(f"[lab] N={N} d={d} rows={len(rows)} " + " ".join(
        f"{k}:ok={r['ok']},mism={r['mismatches']},ratio={r['maxRatio']:.3g}" for k, r in res.items()), flush=True)
    assert res["fused"]["ok"], res["fused"]
    assert res["unfused"]["ok"], res["unfused"]
    assert not res["broken"]["ok"], res["broken"]
    # the unfused kernels also write P into the workspace; O must be finite everywhere
    for o in out.values():
        assert np.isfinite(o).all()


@pytest.mark.parametrize("d", I.LAB_WIDTHS)
def test_control_equals_fused_within_one_key_block(d):
    c = I.lab_case(32, d, seed=5)
    out = run_kinds(c)
    ref, bound = checker.reference_and_bound(c.q[0, :, 0, :], c.k[0, :, 0, :], c.v[0, :, 0, :], c.scale)
    assert np.array_equal(out["broken"], out["fused"])
    for kind in out:
        assert checker.check(out[kind], ref, bound)["ok"], kind


@pytest.mark.parametrize("causal", [False, True])
def test_unfused_matches_oracle_on_ragged_heads(causal):
    # several heads, a ragged T and a causal mask: the unfused path against the definition
    from oracle import attention as oracle
    c = I.make_case("unfused_ragged", 2, 3, 150, 32, I.F32, causal, 21)
    q, k, v = (torch.from_numpy(getattr(c, n)).cuda() for n in ("q", "k", "v"))
    o = torch.full(q.shape, float("nan"), device="cuda")
    s = torch.empty((2, 3, 150, 150), device="cuda")
    fa.check(fa.fa_forward_unfused(q, k, v, o, s, 2, 3, 150, 32, c.scale, int(causal), fa.FA_F32, None))
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(2):
        for h in range(3):
            O, _, P = oracle.head_forward(c.head_f64("q", b, h), c.head_f64("k", b, h), c.head_f64("v", b, h), c.scale,
                                          causal)
            worst = max(worst, float(np.abs(o[b, :, h].cpu().numpy() - O).max()))
            assert float(np.abs(s[b, h].cpu().numpy() - P).max()) <= 2e-6
    assert worst <= 2e-5, worst
