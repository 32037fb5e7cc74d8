"""A whole training step (fa_forward, then fa_backward_nows) captured into a HIP
graph and replayed, through the C ABI (needs an MI355X).

At B16 H16 T512 hd64 the forward has enough query tiles to fill the GPU, so it
never splits keys and allocates nothing; fa_backward_nows keeps D in the
library's static array, so the captured step holds kernel launches only.  Each
replay starts from NaN-filled outputs, with an eager step on another stream
between replays, and must reproduce the eager step's outputs bit for bit.
"""
import pytest
import torch

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import inputs as I

from gpu_util import to_device

pytestmark = pytest.mark.gpu


def test_forward_backward_step_replays_under_graph_capture():
    B, H, T, hd = 16, 16, 512, 64
    c = I.make_case("graph_step", B, H, T, hd, I.BF16, True, 97)
    assert fa.fa_forward_auto_splits(B, H, T, hd, 1, fa.FA_BF16, fa.FA_PREC_BF16) == 1
    q, k, v, do = (to_device(c, n) for n in ("q", "k", "v", "do"))
    shp, lshp = (B, T, H, hd), (B, H, T)

    def outputs():
        return {n: torch.full(lshp if n == "L" else shp, float("nan"), device="cuda")
                for n in ("O", "L", "dQ", "dK", "dV")}

    def step(out, stream):
        fa.check(fa.fa_forward(q, k, v, out["O"], out["L"], B, H, T, hd, c.scale, 1, fa.FA_BF16, fa.FA_PREC_BF16,
                               stream))
        fa.check(fa.fa_backward_nows(q, k, v, out["O"], out["L"], do, out["dQ"], out["dK"], out["dV"], B, H, T, hd,
                                     c.scale, 1, fa.FA_BF16, fa.FA_PREC_BF16, stream))

    print("[graph] eager step", flush=True)
    eager_stream = torch.cuda.Stream()
    ref = outputs()
    step(ref, eager_stream)
    torch.cuda.synchronize()
    assert all(not torch.isnan(t).any() for t in ref.values())

    print("[graph] capture", flush=True)
    cap_stream = torch.cuda.Stream()
    out = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        step(out, cap_stream)
    for rep in range(3):
        print(f"[graph] replay {rep}", flush=True)
        for t in out.values():
            t.fill_(float("nan"))
        other = outputs()
        step(other, eager_stream)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in out:
            assert torch.equal(out[n], ref[n]), (rep, n)
            assert torch.equal(other[n], ref[n]), (rep, n)
