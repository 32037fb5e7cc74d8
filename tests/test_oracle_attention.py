"""Pins of the float64 oracle's attention forward and backward (CPU only).

Each test checks the oracle against something other than its own formula: a
closed form, a hand-expanded tiny case, brute force in plain Python, an
invariance of the mathematics, or central finite differences.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import attention as A


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one_and_mask(causal):
    q, k, v = rnd((9, 5), 1), rnd((9, 5), 2), rnd((9, 5), 3)
    _, _, p = A.head_forward(q, k, v, 0.4, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(9, 1)] == 0.0)
        assert np.all(p[np.tril_indices(9)] > 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_single_position(causal):
    # T = 1: the only key is the query's own; O = V and L = scale <q, k>.
    q, k, v = rnd((1, 1, 1, 6), 4), rnd((1, 1, 1, 6), 5), rnd((1, 1, 1, 6), 6)
    O, L = A.forward(q, k, v, 0.3, causal)
    np.testing.assert_allclose(O, v, atol=1e-15)
    assert L[0, 0, 0] == pytest.approx(0.3 * float(q.ravel() @ k.ravel()), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    # Q = 0: every visible score is 0, so attention is a uniform average.
    T, hd = 7, 3
    q = np.zeros((1, T, 1, hd))
    k, v = rnd((1, T, 1, hd), 7), rnd((1, T, 1, hd), 8)
    O, L = A.forward(q, k, v, 0.5, causal)
    for i in range(T):
        n = i + 1 if causal else T
        np.testing.assert_allclose(O[0, i, 0], v[0, :n, 0].mean(axis=0), atol=1e-14)
        assert L[0, 0, i] == pytest.approx(math.log(n), abs=1e-14)


def test_two_positions_by_hand():
    # T = 2, hd = 1, causal, written out: row 0 sees key 0; row 1 sees keys 0 and 1.
    q = np.array([0.3, -1.2]).reshape(1, 2, 1, 1)
    k = np.array([0.7, 2.0]).reshape(1, 2, 1, 1)
    v = np.array([5.0, -3.0]).reshape(1, 2, 1, 1)
    s = 0.9
    O, L = A.forward(q, k, v, s, True)
    a, b = s * (-1.2) * 0.7, s * (-1.2) * 2.0
    o1 = (math.exp(a) * 5.0 + math.exp(b) * -3.0) / (math.exp(a) + math.exp(b))
    assert O[0, 0, 0, 0] == pytest.approx(5.0, abs=1e-15)
    assert O[0, 1, 0, 0] == pytest.approx(o1, abs=1e-14)
    assert L[0, 0, 0] == pytest.approx(s * 0.3 * 0.7, abs=1e-15)
    assert L[0, 0, 1] == pytest.approx(math.log(math.exp(a) + math.exp(b)), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_loops(causal):
    # Plain Python loops over a tiny problem: scores, safe softmax, weighted sum.
    B, T, H, hd, scale = 2, 5, 2, 3, 0.7
    q, k, v = rnd((B, T, H, hd), 9), rnd((B, T, H, hd), 10), rnd((B, T, H, hd), 11)
    O, L = A.forward(q, k, v, scale, causal)
    for b, h, i in itertools.product(range(B), range(H), range(T)):
        js = range(i + 1) if causal else range(T)
        s = [scale * sum(q[b, i, h, c] * k[b, j, h, c] for c in range(hd)) for j in js]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = sum(w)
        for c in range(hd):
            ref = sum(wj * v[b, j, h, c] for wj, j in zip(w, js)) / z
            assert O[b, i, h, c] == pytest.approx(ref, abs=1e-13)
        assert L[b, h, i] == pytest.approx(mx + math.log(z), abs=1e-13)


def test_layout_heads_and_batches_are_independent():
    # [B, T, H, hd]: head h of batch b only uses q/k/v[b, :, h, :].
    B, T, H, hd = 2, 6, 3, 4
    q, k, v = rnd((B, T, H, hd), 12), rnd((B, T, H, hd), 13), rnd((B, T, H, hd), 14)
    O, L = A.forward(q, k, v, 0.5, True)
    for b, h in itertools.product(range(B), range(H)):
        o1, l1, _ = A.head_forward(q[b, :, h], k[b, :, h], v[b, :, h], 0.5, True)
        np.testing.assert_allclose(O[b, :, h], o1, atol=0)
        np.testing.assert_allclose(L[b, h], l1, atol=0)
    # permuting heads permutes outputs
    perm = [2, 0, 1]
    O2, L2 = A.forward(q[:, :, perm], k[:, :, perm], v[:, :, perm], 0.5, True)
    np.testing.assert_allclose(O2, O[:, :, perm], atol=1e-15)
    np.testing.assert_allclose(L2, L[:, perm], atol=1e-15)


def test_causal_row_equals_truncated_problem():
    # Causal row i equals the last row of the unmasked problem on positions 0..i.
    T, hd = 8, 4
    q, k, v = rnd((1, T, 1, hd), 15), rnd((1, T, 1, hd), 16), rnd((1, T, 1, hd), 17)
    O, L = A.forward(q, k, v, 0.6, True)
    for i in range(T):
        Ot, Lt = A.forward(q[:, :i + 1], k[:, :i + 1], v[:, :i + 1], 0.6, False)
        np.testing.assert_allclose(O[0, i], Ot[0, i], atol=1e-14)
        assert L[0, 0, i] == pytest.approx(Lt[0, 0, i], abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariances(causal):
    T, hd = 7, 3
    q, k, v = rnd((1, T, 1, hd), 18), rnd((1, T, 1, hd), 19), rnd((1, T, 1, hd), 20)
    c = rnd(hd, 21)
    O, L = A.forward(q, k, v, 0.8, causal)
    Ov, Lv = A.forward(q, k, v + c, 0.8, causal)
    np.testing.assert_allclose(Ov, O + c, atol=1e-13)
    np.testing.assert_allclose(Lv, L, atol=0)
    Ok, Lk = A.forward(q, k + c, v, 0.8, causal)
    np.testing.assert_allclose(Ok, O, atol=1e-13)
    np.testing.assert_allclose(Lk[0, 0], L[0, 0] + 0.8 * (q[0, :, 0] @ c), atol=1e-13)


def loss(q, k, v, w, scale, causal):
    O, _ = A.forward(q, k, v, scale, causal)
    return float((O * w).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    # d/dx of sum(O * W) by central differences equals the analytic gradient with dO = W.
    B, T, H, hd, scale = 1, 6, 2, 3, 0.45
    q, k, v, w = (rnd((B, T, H, hd), s) for s in (22, 23, 24, 25))
    dQ, dK, dV, _ = A.backward(q, k, v, w, scale, causal)
    eps = 1e-6
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"], w, scale, causal)
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"], w, scale, causal)
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=1e-6, err_msg=name)


def test_backward_single_position():
    # T = 1: O = V, so dV = dO and dQ = dK = 0.
    q, k, v, do = (rnd((1, 1, 2, 4), s) for s in (26, 27, 28, 29))
    dQ, dK, dV, _ = A.backward(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(dV, do, atol=1e-15)
    np.testing.assert_allclose(dQ, 0, atol=1e-15)
    np.testing.assert_allclose(dK, 0, atol=1e-15)


def test_backward_zero_queries_closed_form():
    # Q = 0 (causal): dK = 0 and dV_j = sum_{i >= j} dO_i / (i + 1).
    T, hd = 6, 3
    q = np.zeros((1, T, 1, hd))
    k, v, do = rnd((1, T, 1, hd), 30), rnd((1, T, 1, hd), 31), rnd((1, T, 1, hd), 32)
    dQ, dK, dV, _ = A.backward(q, k, v, do, 0.7, True)
    np.testing.assert_allclose(dK, 0, atol=1e-15)
    for j in range(T):
        ref = sum(do[0, i, 0] / (i + 1) for i in range(j, T))
        np.testing.assert_allclose(dV[0, j, 0], ref, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    B, T, H, hd = 2, 9, 2, 4
    q, k, v, do = (rnd((B, T, H, hd), s) for s in (33, 34, 35, 36))
    O, _ = A.forward(q, k, v, 0.5, causal)
    dQ, dK, dV, D = A.backward(q, k, v, do, 0.5, causal)
    # rows of dS sum to zero => keys' gradients sum to zero
    np.testing.assert_allclose(dK.sum(axis=1), 0, atol=1e-13)
    # rows of P sum to one => value gradients sum to the upstream gradients
    np.testing.assert_allclose(dV.sum(axis=1), do.sum(axis=1), atol=1e-13)
    # the pre-pass identity D_i = <dO_i, O_i>
    np.testing.assert_allclose(D, np.einsum("bthd,bthd->bht", do, O), atol=1e-13)


def test_flops_convention():
    f = A.flops(64, 16, 1024, 64, True)
    assert f["fwd"] == 4 * 64 * 64 * 16 * 1024 * 1024 / 2
    assert f["total"] == pytest.approx(481.036e9, rel=1e-5)


def test_causal_head_decomposes_into_single_query_problems():
    """A causal row i is the unmasked single-query problem on keys 0..i; dK and dV are the sums of those
    problems' gradients over the rows (the loss is a sum over rows).  The long-sequence GPU test relies on
    this to check rows and key columns of heads too long for the full-head oracle."""
    from exact_attention_forward_amd import inputs as I

    c = I.make_case("decomp", 1, 1, 96, 16, I.F32, True, 5)
    q, k, v, do = (c.head_f64(n, 0, 0) for n in ("q", "k", "v", "do"))
    O, L, _ = A.head_forward(q, k, v, c.scale, True)
    dQ, dK, dV, _ = A.head_backward(q, k, v, do, c.scale, True)
    dK_sum, dV_sum = np.zeros_like(dK), np.zeros_like(dV)
    for i in range(96):
        o, l, _ = A.head_forward(q[i:i + 1], k[:i + 1], v[:i + 1], c.scale, False)
        dq, dk, dv, _ = A.head_backward(q[i:i + 1], k[:i + 1], v[:i + 1], do[i:i + 1], c.scale, False)
        np.testing.assert_allclose(o[0], O[i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[0], L[i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dq[0], dQ[i], rtol=0, atol=1e-13)
        dK_sum[:i + 1] += dk
        dV_sum[:i + 1] += dv
    np.testing.assert_allclose(dK_sum, dK, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV_sum, dV, rtol=0, atol=1e-12)
