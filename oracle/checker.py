"""Per-element error bound and checker of the fused-attention lesson, float64.

Test infrastructure (see the package docstring).

The "Lesson K23, fused attention" facts page (block ``correctness``, field
``about``) checks every output O_ic of a float32 kernel against a float64
reference of standard softmax attention with the max subtracted, with the
tolerance

    bound_ic = 2 (exp(2 delta_i + 2 e_i) - 1 + gamma_K) sum_j p_ij |v_jc| + floor,

where delta is the score error of a length-d dot product times the scale
(gamma_(d+1) scale sum_k |q_ik k_jk|, Higham's bound for a computed dot
product), e is the accuracy of the float32 exponential ((3 + 2|x|) ulp for an
argument x), gamma_K is the error of the length-K sums over keys, and floor
covers underflow.  The page gives no formula for the floor nor says whether
delta and e are taken per score or per row; the readings here (largest per
row; floor = K 2^-126 max_j |v_jc|) are listed with the other readings of the
pages.  A checked output passes when |out - ref| <= bound; a run passes when
no checked output fails (block ``lab``: every row up to N = 1024, the first 64
rows above).

The lesson's own controls of the checker (block ``controls.checker``) pin
this module: a tiled float32 output passes, the exact answer rounded to
float32 passes, one output moved by 0.001 fails with exactly one mismatch,
and zero tolerance rejects a float32 output.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24    # float32 unit roundoff
ULP = 2.0 ** -23  # float32 spacing of numbers in [1, 2)


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u) for float32."""
    return n * U / (1.0 - n * U)


def rows_checked(N: int) -> np.ndarray:
    """Rows the lab checks: all of them up to N = 1024, the first 64 above."""
    return np.arange(N) if N <= 1024 else np.arange(64)


def reference_and_bound(q, k, v, scale: float, rows=None, causal: bool = False):
    """One head.  q, k, v: [N, d] (the exact stored values).

    Returns (ref [R, d], bound [R, d]) for the given rows (default: all).
    With ``causal`` row i sees keys j <= i only, and every term of the bound
    is taken over those keys: K is the count of visible keys, delta and e their
    largest values, the floor their largest |v|.  Row i of the causal bound is
    therefore the unmasked bound of the problem truncated to keys 0..i.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    vis = np.arange(N)[None, :] <= rows[:, None] if causal else np.ones((len(rows), N), bool)
    s = np.where(vis, scale * (q[rows] @ k.T), -np.inf)
    m = s.max(axis=1)
    x = s - m[:, None]
    w = np.where(vis, np.exp(x), 0.0)
    p = w / w.sum(axis=1)[:, None]
    ref = p @ v
    delta = np.where(vis, gamma(d + 1) * scale * (np.abs(q[rows]) @ np.abs(k).T), 0.0)
    e = np.where(vis, (3.0 + 2.0 * np.abs(np.where(vis, x, 0.0))) * ULP, 0.0)
    K = vis.sum(axis=1)
    fac = 2.0 * (np.exp(2.0 * delta.max(axis=1) + 2.0 * e.max(axis=1)) - 1.0 + np.array([gamma(int(n)) for n in K]))
    vmax = np.array([np.abs(v[vis[r]]).max(axis=0) for r in range(len(rows))])
    floor = K[:, None] * 2.0 ** -126 * vmax
    bound = fac[:, None] * (p @ np.abs(v)) + floor
    return ref, bound


def check(out, ref, bound) -> dict:
    """Checker result: ok, mismatches, outputs, maxErr, maxRatio (largest error over its bound)."""
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref)
    bad = ~(err <= bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    n = int(np.count_nonzero(bad))
    return {"ok": n == 0, "mismatches": n, "outputs": int(out.size), "maxErr": float(np.nanmax(err)),
            "maxRatio": float(np.nanmax(ratio))}
