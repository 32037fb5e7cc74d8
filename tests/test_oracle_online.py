"""Pins of the oracle's online normaliser, merge and block-wise forward (CPU only).

Fixtures under tests/golden/ hold values printed on the "Lesson K23, fused
attention" facts page (blocks controls.vector and probe.heads).
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest

from oracle import attention as A
from oracle import online as ON

GOLD = Path(__file__).resolve().parent / "golden"


def test_page_vector_trace():
    g = json.loads((GOLD / "online_vector.json").read_text())
    tr = ON.normaliser_trace(g["values"])
    for (m, l), ref in zip(tr, g["trace"]):
        assert m == ref["m"]
        assert l == pytest.approx(ref["l"], abs=5e-5)  # printed to 4 decimals
    assert tr[-1][1] == pytest.approx(g["sum"], abs=5e-5)
    rises = sum(1 for a, b in zip(tr, tr[1:]) if b[0] > a[0])
    assert rises == g["maxRises"]
    # online weights exp(x - m_final) / l_final against the two-pass safe softmax
    m, l = tr[-1]
    w_online = np.exp(np.array(g["values"]) - m) / l
    assert np.abs(w_online - ON.softmax_two_pass(g["values"])).max() <= 4 * g["maxWeightDiff"]


def test_page_broken_trace():
    g = json.loads((GOLD / "online_vector.json").read_text())
    tr = ON.broken_trace(g["values"])
    for (m, l), ref in zip(tr, g["brokenTrace"]):
        assert m == ref["m"]
        assert l == pytest.approx(ref["l"], abs=5e-5)
    assert tr[-1][1] == pytest.approx(g["brokenSum"], abs=5e-5)
    # the block recurrence with one-element blocks is the element recurrence
    assert ON.block_trace(g["values"], 1, rescale=False)[-1][1] == pytest.approx(tr[-1][1], abs=1e-12)
    assert ON.block_trace(g["values"], 1)[-1][1] == pytest.approx(ON.normaliser_trace(g["values"])[-1][1], abs=1e-12)


def test_page_probe_tile_traces():
    # Scores printed to 4 decimals, so traces agree to about 1.5e-4.
    g = json.loads((GOLD / "probe_traces.json").read_text())
    for head in g["heads"]:
        row = head["row"]
        assert max(row) == head["rowMax"] and int(np.argmax(row)) == head["argmax"]
        tr = ON.block_trace(row, 4)
        assert len(tr) == len(head["trace"])
        for (m, l), ref in zip(tr, head["trace"]):
            assert m == pytest.approx(ref["m"], abs=1e-12)
            assert l == pytest.approx(ref["l"], abs=1.5e-4)


def test_merge_is_associative_and_commutative():
    rng = np.random.default_rng(40)
    s = rng.standard_normal(50) * 3
    v = rng.standard_normal((50, 4))
    whole = ON.state(s, v)
    for trial in range(20):
        cuts = sorted(rng.choice(np.arange(1, 50), size=rng.integers(1, 8), replace=False))
        parts = [ON.state(s[a:b], v[a:b]) for a, b in zip([0, *cuts], [*cuts, 50])]
        # left fold, right fold and a shuffled fold
        lf = parts[0]
        for p in parts[1:]:
            lf = ON.merge(lf, p)
        rf = parts[-1]
        for p in reversed(parts[:-1]):
            rf = ON.merge(p, rf)
        order = rng.permutation(len(parts))
        sf = parts[order[0]]
        for i in order[1:]:
            sf = ON.merge(sf, parts[i])
        for st in (lf, rf, sf):
            assert st[0] == whole[0]
            assert st[1] == pytest.approx(whole[1], rel=1e-14)
            np.testing.assert_allclose(st[2], whole[2], rtol=1e-13, atol=1e-14)
    o, L = ON.finish(whole)
    np.testing.assert_allclose(o, ON.softmax_two_pass(s) @ v, atol=1e-14)
    assert L == pytest.approx(np.log(np.exp(s).sum()), abs=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,br,bc", [(16, 16, 16), (8, 16, 16), (20, 16, 16), (37, 8, 5), (64, 16, 64), (33, 32, 4)])
def test_tiled_forward_equals_definition(causal, T, br, bc):
    rng = np.random.default_rng(T * 7 + br)
    q, k, v = (rng.standard_normal((T, 6)) for _ in range(3))
    O, L, _ = A.head_forward(q, k, v, 0.5, causal)
    Ot, Lt = ON.tiled_forward(q, k, v, 0.5, causal, br, bc)
    np.testing.assert_allclose(Ot, O, atol=1e-13)
    np.testing.assert_allclose(Lt, L, atol=1e-13)


def test_broken_rescale_fails_iff_rows_span_blocks():
    rng = np.random.default_rng(41)
    q, k, v = (rng.standard_normal((64, 16)) * 2 for _ in range(3))
    O, _, _ = A.head_forward(q, k, v, 0.25, False)
    one, _ = ON.tiled_forward(q, k, v, 0.25, False, 64, 64, rescale=False)
    np.testing.assert_allclose(one, O, atol=1e-13)  # a single block never rescales
    many, _ = ON.tiled_forward(q, k, v, 0.25, False, 64, 16, rescale=False)
    assert np.abs(many - O).max() > 1e-2
