"""fa_backward_nows (the backward whose D workspace is the library's static
device array) against fa_backward with a caller workspace, through the C ABI
(needs an MI355X).

Two calls in a row on each path, the second smaller than the first, so the
second call runs on the array the first one left behind.  Same kernels and
the same D, so the results must be bitwise equal; they are also held to the
oracle's bar.
"""
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I

from gpu_util import BF16_TOL, F32_TOL, assert_within, full_errors, run_case, to_device

pytestmark = pytest.mark.gpu

# (dtype, hd, causal, prec): the fused-D dQ stage (bf16 hd 64), the D pre-pass
# (bf16 hd 128, float32)
PATHS = [(I.BF16, 64, True, fa.FA_PREC_BF16), (I.BF16, 128, True, fa.FA_PREC_BF16X2), (I.F32, 32, False, 0)]


@pytest.mark.parametrize("dtype,hd,causal,prec", PATHS, ids=lambda x: str(x))
def test_static_workspace_backward_equals_fa_backward(dtype, hd, causal, prec):
    cases = [I.make_case("nows_big", 2, 4, 333, hd, dtype, causal, 51 + hd),
             I.make_case("nows_small", 1, 3, 77, hd, dtype, causal, 52 + hd)]
    dtc = {I.BF16: fa.FA_BF16, I.F32: fa.FA_F32}[dtype]
    for c in cases:
        print(f"[nows] {c.name} B{c.B} H{c.H} T{c.T} hd{hd} {dtype} causal={causal} prec={prec}", flush=True)
        ref = run_case(c, prec)
        q, k, v, do = (to_device(c, n) for n in ("q", "k", "v", "do"))
        B, T, H, _ = q.shape
        dq, dk, dv = (torch.full_like(ref["dQ"], float("nan")) for _ in range(3))
        fa.check(fa.fa_backward_nows(q, k, v, ref["O"], ref["L"], do, dq, dk, dv, B, H, T, hd, c.scale, causal, dtc,
                                     prec, None))
        torch.cuda.synchronize()
        for n, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert torch.equal(t, ref[n]), (c.name, n)
        got = dict(ref)
        got.update(dQ=dq, dK=dk, dV=dv)
        assert_within(full_errors(c, got), F32_TOL if dtype == I.F32 else BF16_TOL, c.name)


def test_static_workspace_backward_rejects_oversize_before_launch():
    x = torch.zeros(16, device="cuda")
    p = x.data_ptr()
    st = fa.fa_backward_nows(p, p + 1 * 2**30, p + 2 * 2**30, p + 3 * 2**30, p + 4 * 2**30, p + 5 * 2**30,
                             p + 6 * 2**30, p + 7 * 2**30, p + 8 * 2**30, 1, 1, (1 << 22) + 1, 8, 0.3, 1, fa.FA_F32, 0,
                             None)
    assert st == fa.FA_ERR_TOO_LARGE
