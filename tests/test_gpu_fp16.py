"""IEEE half inputs on the GPU, and the overflow of the softmax without its max.

Parity: the forward and the backward with FA_F16 inputs against the float64
oracle (max abs 2e-2, the 16-bit input bar), through the C ABI, on small shapes
and on a ragged shape where every persistent workgroup walks several tiles.

Overflow ("Lesson K23, fused attention", block ``overflow``): scores reaching
ln 65520 = 11.09 are harmless for fa_forward, which subtracts the running max,
but the control fa_forward_nomax (no max subtracted, weights entering P.V as
binary16) turns exactly the rows whose largest visible score reaches the
threshold non-finite; with float32 inputs the same control stays finite there
(float32 overflows only above 88.7).
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I
from oracle import attention as oracle
from oracle import overflow

from gpu_util import BF16_TOL, assert_within, full_errors, head_errors, run_case, to_device

pytestmark = pytest.mark.gpu

SHAPES = [(1, 2, 300, 64), (2, 1, 129, 128), (1, 1, 1024, 64), (1, 3, 33, 64), (1, 2, 191, 64), (2, 1, 130, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}T{}hd{}".format(*s))
def test_f16_forward_backward(shape, causal):
    B, H, T, hd = shape
    c = I.make_case("f16", B, H, T, hd, I.F16, causal, 500 + T + hd)
    err = full_errors(c, run_case(c))
    print(f"[f16] {shape} causal={causal} " + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert_within(err, BF16_TOL, c.name)


@pytest.mark.parametrize("causal", [True, False])
def test_f16_ragged_multi_item_sampled(causal):
    # enough (tile, head) items that every persistent workgroup walks several
    B, H, T, hd = 2, 128, 1000, 64
    c = I.make_case("f16_multi_item", B, H, T, hd, I.F16, causal, 71)
    out = run_case(c)
    for n, t in out.items():
        assert bool(torch.isfinite(t).all()), f"{n} has unwritten or non-finite elements"
    worst = {}
    for b, h in [(0, 0), (0, 37), (1, 64), (1, 127)]:
        for n, e in head_errors(c, out, b, h).items():
            worst[n] = max(worst.get(n, 0.0), e)
    print(f"[f16 multi-item] causal={causal} " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    assert_within(worst, BF16_TOL, c.name)


def test_f16_splitkv():
    c = I.make_case("f16_split", 1, 2, 700, 64, I.F16, True, 7)
    q, k, v = (to_device(c, n) for n in ("q", "k", "v"))
    o = torch.empty((1, 700, 2, 64), device="cuda")
    lse = torch.empty((1, 2, 700), device="cuda")
    ws = torch.empty((5 * (700 * 2 * 64 + 2 * 700),), device="cuda")
    fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, ws, 1, 2, 700, 64, c.scale, 1, 5, fa.FA_F16, 0, None))
    torch.cuda.synchronize()
    for h in range(2):
        O, L, _ = oracle.head_forward(c.head_f64("q", 0, h), c.head_f64("k", 0, h), c.head_f64("v", 0, h), c.scale,
                                      True)
        assert float(np.abs(o[0, :, h].cpu().numpy() - O).max()) <= BF16_TOL
        assert float(np.abs(lse[0, h].cpu().numpy() - L).max()) <= BF16_TOL


def large_score_case(dtype):
    # q scaled by 4: about half of the 256 rows reach a largest score of 11.09
    c = I.make_case("f16_large", 1, 1, 256, 64, I.F32, False, 11)
    q = (c.q.astype(np.float64) * 4.0).astype(np.float32)
    if dtype == I.F16:
        c.q, c.k, c.v = (a.astype(np.float16).view(np.uint16) for a in (q, c.k, c.v))
        c.dtype = I.F16
    else:
        c.q = q
    return c


@pytest.mark.parametrize("dtype", [I.F16, I.F32])
def test_softmax_without_max_overflows_in_half(dtype):
    c = large_score_case(dtype)
    qd, kd, vd = (to_device(c, n) for n in ("q", "k", "v"))
    dt = fa.FA_F16 if dtype == I.F16 else fa.FA_F32
    T, hd = c.T, c.hd
    outs = {}
    for name, fn in (("safe", fa.fa_forward), ("nomax", fa.fa_forward_nomax)):
        o = torch.full((1, T, 1, hd), float("nan"), device="cuda")
        lse = torch.full((1, 1, T), float("nan"), device="cuda")
        if name == "safe":
            fa.check(fn(qd, kd, vd, o, lse, 1, 1, T, hd, c.scale, 0, dt, 0, None))
        else:
            fa.check(fn(qd, kd, vd, o, lse, 1, 1, T, hd, c.scale, 0, dt, None))
        torch.cuda.synchronize()
        outs[name] = o[0, :, 0].cpu().numpy()
    q, k, v = (c.head_f64(n, 0, 0) for n in ("q", "k", "v"))
    O, _, _ = oracle.head_forward(q, k, v, c.scale, False)
    smax = (c.scale * q @ k.T).max(axis=1)
    over = smax > overflow.THRESHOLD + 1e-3
    under = smax < overflow.THRESHOLD - 1e-3
    assert over.sum() >= 10 and under.sum() >= 10, (over.sum(), under.sum())
    # the safe forward is right everywhere
    assert np.isfinite(outs["safe"]).all()
    assert float(np.abs(outs["safe"] - O).max()) <= (BF16_TOL if dtype == I.F16 else 2e-5)
    bad = ~np.isfinite(outs["nomax"]).all(axis=1)
    print(f"[overflow] {dtype}: rows over threshold {int(over.sum())}, non-finite rows {int(bad.sum())}", flush=True)
    if dtype == I.F16:
        assert bad[over].all(), "every row reaching ln 65520 overflows without the max"
        assert not bad[under].any()
        assert float(np.abs(outs["nomax"][under] - O[under]).max()) <= BF16_TOL
    else:
        assert not bad.any()
        assert float(np.abs(outs["nomax"] - O).max()) <= 1e-4
