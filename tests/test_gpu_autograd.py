"""The autograd operation (api.attention) runs the same two C entry points as the direct calls.

Its output and gradients are compared bit for bit with fa_forward / fa_backward
called directly on the same inputs (the kernels are deterministic), and for
float32 inputs also with the float64 oracle ("Flash Attention 2 -- backward
pass notes", section "The math (FA2 backward with recompute)").
"""
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import api
from exact_attention_forward_amd import inputs as I
from gpu_util import F32_TOL, assert_within, heads_errors, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,prec", [(I.F32, fa.FA_PREC_DEFAULT), (I.BF16, fa.FA_PREC_BF16),
                                        (I.BF16, fa.FA_PREC_BF16X2)])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_autograd_equals_direct_calls(dtype, prec, causal):
    c = I.make_case("autograd", 2, 3, 200, 64, dtype, causal, 31)
    q, k, v, do = (to_device(c, n) for n in ("q", "k", "v", "do"))
    print(f"[autograd] {dtype} prec={prec} causal={causal}", flush=True)
    o, lse = api.forward(q, k, v, c.scale, causal, prec)
    dq, dk, dv, delta = api.backward(q, k, v, o, lse, do, c.scale, causal, prec)

    qa, ka, va = (x.clone().requires_grad_() for x in (q, k, v))
    oa = api.attention(qa, ka, va, c.scale, causal, prec)
    oa.backward(do.float())  # rounded back to the inputs' dtype inside, exactly
    torch.cuda.synchronize()
    assert torch.equal(oa.detach(), o)
    for got, want in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        assert got.dtype == q.dtype
        assert torch.equal(got, want.to(q.dtype))

    if dtype == I.F32:
        out = dict(O=oa.detach(), L=lse, dQ=qa.grad, dK=ka.grad, dV=va.grad, D=delta)
        err = heads_errors(c, out, [(0, 0), (1, 2)])
        assert_within(err, F32_TOL, "autograd float32")
