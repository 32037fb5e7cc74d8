"""Exact scaled-dot-product attention and its gradient, float64, by definition.

Test infrastructure (see the package docstring): a plain, slow, obviously
correct implementation.  Per (batch, head), with i, j in [0, T):

* s_ij = scale * <q_i, k_j>  -- "Flash Attention 2 -- forward pass notes",
  section "The algorithm" (S = Q K^T / sqrt(d), the caller passes scale);
* visible set V(i) = {j <= i} for the causal mask (diagonal kept), else all j
  -- same section (causal_mask sets S_ij to -inf for j > i);
* L_i = m_i + ln sum_{j in V(i)} exp(s_ij - m_i) with m_i the row maximum (the
  log-sum-exp the forward saves, "Flash Attention 2 -- backward pass notes",
  section "The math (FA2 backward with recompute)");
* P_ij = exp(s_ij - L_i) on V(i), 0 elsewhere; O_i = sum_j P_ij v_j;
* backward, the textbook softmax Jacobian (same section of the backward notes):
  dV_j = sum_i P_ij dO_i; dP_ij = <dO_i, v_j>; D_i = sum_j P_ij dP_ij;
  dS_ij = P_ij (dP_ij - D_i); dQ_i = scale sum_j dS_ij k_j;
  dK_j = scale sum_i dS_ij q_i.

D is computed from P and dP here, not from <dO_i, O_i>, so the identity the
backward notes use for the pre-pass is itself checked by the tests.

Layout: q, k, v, dO, O, dQ, dK, dV are [B, T, H, hd]; L and D are [B, H, T].
The score matrix of one head is materialised whole (no tiling, no online
merge, no base-2 exponentials).
"""
from __future__ import annotations

import numpy as np


def _scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    s = scale * (q @ k.T)
    if causal:
        T = s.shape[0]
        s[np.triu_indices(T, 1)] = -np.inf
    return s


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool):
    """One head: q, k, v [T, hd] -> (O [T, hd], L [T], P [T, T])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = _scores(q, k, scale, causal)
    m = s.max(axis=1)
    L = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - L[:, None])
    return p @ v, L, p


def head_backward(q, k, v, do, scale: float, causal: bool):
    """One head: returns (dQ, dK, dV, D) for the upstream gradient dO = d loss / d O."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    _, _, p = head_forward(q, k, v, scale, causal)
    dv = p.T @ do
    dp = do @ v.T
    D = (p * dp).sum(axis=1)
    ds = p * (dp - D[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, D


def forward(q, k, v, scale: float, causal: bool):
    """q, k, v [B, T, H, hd] -> (O [B, T, H, hd] float64, L [B, H, T] float64)."""
    B, T, H, hd = q.shape
    O = np.empty((B, T, H, hd))
    L = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            O[b, :, h, :], L[b, h, :], _ = head_forward(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], scale, causal)
    return O, L


def backward(q, k, v, do, scale: float, causal: bool):
    """Returns (dQ, dK, dV [B, T, H, hd], D [B, H, T]), all float64."""
    B, T, H, hd = q.shape
    dQ = np.empty((B, T, H, hd))
    dK = np.empty((B, T, H, hd))
    dV = np.empty((B, T, H, hd))
    D = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            r = head_backward(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :], scale, causal)
            dQ[b, :, h, :], dK[b, :, h, :], dV[b, :, h, :], D[b, h, :] = r
    return dQ, dK, dV, D


def flops(B: int, H: int, T: int, hd: int, causal: bool) -> dict:
    """Counted floating-point work of one forward + backward.

    Forward 4*hd per (query, visible key) pair (two length-hd products, S and
    PV); backward 10*hd per pair (dV, dP, dQ, dK and the recomputed S).  The
    causal pair count is T^2/2, i.e. the full count halved.
    """
    pairs = B * H * T * T * (0.5 if causal else 1.0)
    return {"fwd": 4.0 * hd * pairs, "bwd": 10.0 * hd * pairs, "total": 14.0 * hd * pairs, "pairs": pairs}
