"""Split-key forward (fa_forward_splitkv) against the float64 oracle, through the C ABI.

Each key range produces a partial (O_s, L_s); the merge kernel combines them
(forward notes, the merge after the loop).  The merged O and L must meet the
same bars as fa_forward (max abs 2e-5 for float32 inputs, 2e-2 for bfloat16),
for split counts that leave empty, partial and causal-skipped ranges.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I
from oracle import attention as oracle

from gpu_util import BF16_TOL, F32_TOL, to_device

pytestmark = pytest.mark.gpu


def run_split(c, nsplit, prec=fa.FA_PREC_DEFAULT):
    q, k, v = (to_device(c, n) for n in ("q", "k", "v"))
    B, T, H, hd = q.shape
    o = torch.full((B, T, H, hd), float("nan"), device="cuda")
    lse = torch.full((B, H, T), float("nan"), device="cuda")
    ws = torch.full((nsplit * (B * T * H * hd + B * H * T),), float("nan"), device="cuda")
    dt = {I.BF16: fa.FA_BF16, I.F16: fa.FA_F16}.get(c.dtype, fa.FA_F32)
    fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, ws, B, H, T, hd, c.scale, int(c.causal), nsplit, dt, prec, None))
    torch.cuda.synchronize()
    return o, lse


def oracle_errors(c, o, lse):
    worst = {"O": 0.0, "L": 0.0}
    for b in range(c.B):
        for h in range(c.H):
            O, L, _ = oracle.head_forward(c.head_f64("q", b, h), c.head_f64("k", b, h), c.head_f64("v", b, h), c.scale,
                                          c.causal)
            worst["O"] = max(worst["O"], float(np.abs(o[b, :, h].cpu().numpy() - O).max()))
            worst["L"] = max(worst["L"], float(np.abs(lse[b, h].cpu().numpy() - L).max()))
    return worst


@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 300, 64), (2, 3, 129, 16), (1, 2, 1000, 128)],
                         ids=lambda s: "B{}H{}T{}hd{}".format(*s))
def test_splitkv_f32(shape, causal, nsplit):
    B, H, T, hd = shape
    c = I.make_case("split_f32", B, H, T, hd, I.F32, causal, 300 + T + hd)
    o, lse = run_split(c, nsplit)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    err = oracle_errors(c, o, lse)
    print(f"[split] {shape} causal={causal} nsplit={nsplit} {err}", flush=True)
    assert err["O"] <= F32_TOL and err["L"] <= F32_TOL, err


@pytest.mark.parametrize("prec", [fa.FA_PREC_BF16, fa.FA_PREC_DEFAULT])
@pytest.mark.parametrize("nsplit", [1, 4, 13, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hd", [64, 128])
def test_splitkv_bf16(hd, causal, nsplit, prec):
    # 64 splits of T = 777 round to 32-key chunks: 25 hold keys, the rest are
    # empty and must come out as O = 0, L = -inf partials that the merge skips.
    c = I.make_case("split_bf16", 1, 2, 777, hd, I.BF16, causal, 400 + hd)
    o, lse = run_split(c, nsplit, prec)
    err = oracle_errors(c, o, lse)
    print(f"[split] bf16 hd={hd} causal={causal} nsplit={nsplit} prec={prec} {err}", flush=True)
    assert err["O"] <= BF16_TOL and err["L"] <= BF16_TOL, err


def test_splitkv_agrees_with_fused_on_one_long_head():
    # the case split keys exist for: one head, long T
    c = I.lab_case(4096, 64)
    q, k, v = (torch.from_numpy(getattr(c, n)).cuda() for n in ("q", "k", "v"))
    o1, l1 = torch.empty_like(q), torch.empty((1, 1, 4096), device="cuda")
    fa.check(fa.fa_forward(q, k, v, o1, l1, 1, 1, 4096, 64, c.scale, 0, fa.FA_F32, 0, None))
    o2, l2 = run_split(c, 16)
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-5 and float((l1 - l2).abs().max()) <= 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_auto_split(dt, causal):
    # One head of T = 4096: the plain forward's 32 query tiles would leave most
    # of the GPU idle, so fa_forward splits the keys.  Its result must be the
    # split-key forward's for the count it reports, bit for bit, and meet the
    # oracle bar.
    B, H, T, hd = 1, 1, 4096, 64
    c = I.make_case("auto_split", B, H, T, hd, I.BF16 if dt == "bf16" else I.F32, causal, 77)
    fdt = fa.FA_BF16 if dt == "bf16" else fa.FA_F32
    n = fa.fa_forward_auto_splits(B, H, T, hd, int(causal), fdt, fa.FA_PREC_DEFAULT)
    print(f"[auto split] {dt} causal={causal} nsplit={n}", flush=True)
    assert 2 <= n <= 64
    q, k, v = (to_device(c, x) for x in ("q", "k", "v"))
    o = torch.full((B, T, H, hd), float("nan"), device="cuda")
    lse = torch.full((B, H, T), float("nan"), device="cuda")
    fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, c.scale, int(causal), fdt, fa.FA_PREC_DEFAULT, None))
    o2, l2 = run_split(c, n)
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    err = oracle_errors(c, o, lse)
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    assert err["O"] <= tol and err["L"] <= tol, err


def test_forward_auto_split_leaves_full_workloads_alone():
    # 8192 query tiles at B64 H16 T1024 fill the GPU: no split
    assert fa.fa_forward_auto_splits(64, 16, 1024, 64, 1, fa.FA_BF16, fa.FA_PREC_DEFAULT) == 1
    assert fa.fa_forward_auto_splits(4, 16, 8192, 128, 1, fa.FA_BF16, fa.FA_PREC_BF16X2) == 1


def test_splitkv_without_workspace_is_the_plain_forward():
    # nsplit = 1 and no workspace: the plain forward, bit for bit the unsplit
    # fa_forward of a workload it does not split, and within the oracle bar for
    # one it would split
    c = I.make_case("plain", 8, 16, 1024, 64, I.BF16, True, 5)
    assert fa.fa_forward_auto_splits(8, 16, 1024, 64, 1, fa.FA_BF16, fa.FA_PREC_DEFAULT) == 1
    q, k, v = (to_device(c, x) for x in ("q", "k", "v"))
    o1, l1 = torch.empty(q.shape, device="cuda"), torch.empty((8, 16, 1024), device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa.check(fa.fa_forward(q, k, v, o1, l1, 8, 16, 1024, 64, c.scale, 1, fa.FA_BF16, 0, None))
    fa.check(fa.fa_forward_splitkv(q, k, v, o2, l2, None, 8, 16, 1024, 64, c.scale, 1, 1, fa.FA_BF16, 0, None))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    c1 = I.make_case("plain_one_head", 1, 1, 2048, 64, I.BF16, True, 6)
    q, k, v = (to_device(c1, x) for x in ("q", "k", "v"))
    o = torch.full((1, 2048, 1, 64), float("nan"), device="cuda")
    lse = torch.full((1, 1, 2048), float("nan"), device="cuda")
    fa.check(fa.fa_forward_splitkv(q, k, v, o, lse, None, 1, 1, 2048, 64, c1.scale, 1, 1, fa.FA_BF16, 0, None))
    torch.cuda.synchronize()
    err = oracle_errors(c1, o, lse)
    assert err["O"] <= BF16_TOL and err["L"] <= BF16_TOL, err


def test_forward_auto_split_under_graph_capture():
    # A capture on a stream without a workspace yet cannot allocate one: the
    # captured fa_forward is the plain forward.  After one call on the stream
    # the workspace exists and the captured call splits.  Each graph is
    # replayed three times, with eager work between replays.
    B, H, T, hd = 1, 1, 2048, 64
    c = I.make_case("auto_split_graph", B, H, T, hd, I.BF16, True, 91)
    n = fa.fa_forward_auto_splits(B, H, T, hd, 1, fa.FA_BF16, fa.FA_PREC_DEFAULT)
    assert n >= 2
    q, k, v = (to_device(c, x) for x in ("q", "k", "v"))
    po, pl = torch.empty((B, T, H, hd), device="cuda"), torch.empty((B, H, T), device="cuda")
    fa.check(fa.fa_forward_splitkv(q, k, v, po, pl, None, B, H, T, hd, c.scale, 1, 1, fa.FA_BF16, 0, None))
    so, sl = run_split(c, n)
    for warm in (False, True):
        s = torch.cuda.Stream()
        o = torch.full((B, T, H, hd), float("nan"), device="cuda")
        lse = torch.full((B, H, T), float("nan"), device="cuda")
        if warm:
            fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, c.scale, 1, fa.FA_BF16, 0, s))
            s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fa.check(fa.fa_forward(q, k, v, o, lse, B, H, T, hd, c.scale, 1, fa.FA_BF16, 0, s))
        eo, el = (so, sl) if warm else (po, pl)
        for _ in range(3):
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, eo) and torch.equal(lse, el), f"warm={warm}"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("growing", [False, True], ids=["plain_keys", "growing_keys"])
@pytest.mark.parametrize("causal", [False, True])
def test_streamed_forward_is_the_tile_kernel_bit_for_bit(causal, growing, dt):
    # At hd 64 the plain forward (one split, no workspace) runs the streamed
    # kernel, which skips the row max of a pipelined block and redoes the
    # block with it only when a row-sum increment shows a weight of 2^slack or
    # more; the split forward with one split runs the per-block tile kernel,
    # which takes every block's max, and a merge that returns its one partial
    # unchanged.  Both must give the same bits.  With the keys of the second
    # half scaled by 6, later blocks' scores exceed each row's reference by far
    # more than the slack, so the redo path runs (and raises the reference).
    B, H, T, hd = 2, 3, 700, 64
    bf = dt == "bf16"
    c = I.make_case("streamed_vs_tile", B, H, T, hd, I.BF16 if bf else I.F16, causal, 31)
    if growing:
        k = I.bf16_bits_to_f32(c.k).copy() if bf else c.k.view(np.float16).astype(np.float32)
        k[:, T // 2:] *= 6.0
        c.k = I.f32_to_bf16_bits(k).reshape(c.k.shape) if bf else k.astype(np.float16).view(np.uint16)
    q, k, v = (to_device(c, x) for x in ("q", "k", "v"))
    o1 = torch.full((B, T, H, hd), float("nan"), device="cuda")
    l1 = torch.full((B, H, T), float("nan"), device="cuda")
    code, prec = (fa.FA_BF16, fa.FA_PREC_BF16) if bf else (fa.FA_F16, fa.FA_PREC_DEFAULT)
    fa.check(fa.fa_forward_splitkv(q, k, v, o1, l1, None, B, H, T, hd, c.scale, int(causal), 1, code, prec, None))
    o2, l2 = run_split(c, 1, prec)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    err = oracle_errors(c, o1, l1)
    print(f"[streamed vs tile] {dt} causal={causal} growing={growing} {err}", flush=True)
    assert err["O"] <= BF16_TOL and err["L"] <= BF16_TOL, err
