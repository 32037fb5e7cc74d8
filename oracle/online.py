"""Online softmax normaliser, its merge, and a block-wise attention forward (float64).

Test infrastructure (see the package docstring).

* ``normaliser_trace`` -- Milakov and Gimelshein's online normaliser
  (Algorithm 3 as quoted on the "fused attention" lesson page, block
  ``sources.onlineSoftmax``): m_j = max(m_{j-1}, x_j) and
  d_j = d_{j-1} * exp(m_{j-1} - m_j) + exp(x_j - m_j), from m_0 = -inf, d_0 = 0.
* ``broken_trace`` -- the same recurrence without the exp(m_{j-1} - m_j)
  rescale of the running sum: the lesson page's negative control.
* ``merge`` -- combine two partial states (m, l, o) of disjoint key sets
  ("Flash Attention 2 -- forward pass notes", the merge identity after the
  loop; the lesson page calls the operator associative and commutative).
* ``tiled_forward`` -- the forward loop of the forward notes, section "Loop
  (per (b, h, Q-tile))": for each key block, m_new = max(m, block max),
  alpha = exp(m - m_new), O and l rescaled by alpha, then p = exp(s - m_new)
  accumulated; causal blocks past the tile's last row skipped; finally
  O / l and L = m + ln l.  ``rescale=False`` drops alpha (the broken variant).
"""
from __future__ import annotations

import math

import numpy as np


def normaliser_trace(x):
    """Running (m, d) after each element of x."""
    m, d = -math.inf, 0.0
    out = []
    for xj in x:
        mn = max(m, xj)
        d = d * (math.exp(m - mn) if m != -math.inf else 0.0) + math.exp(xj - mn)
        m = mn
        out.append((m, d))
    return out


def broken_trace(x):
    """Running (m, d) with the rescale of d omitted."""
    m, d = -math.inf, 0.0
    out = []
    for xj in x:
        mn = max(m, xj)
        d = d + math.exp(xj - mn)
        m = mn
        out.append((m, d))
    return out


def block_trace(x, block: int, rescale: bool = True):
    """Running (m, l) after each block of `block` consecutive elements.

    Per block: m_new = max(m, max of block); l = l * exp(m - m_new) + sum exp(x - m_new).
    """
    m, l = -math.inf, 0.0
    out = []
    for s in range(0, len(x), block):
        blk = list(x[s:s + block])
        mn = max(m, max(blk))
        if not rescale:
            a = 1.0
        else:
            a = math.exp(m - mn) if m != -math.inf else 0.0
        l = l * a + sum(math.exp(v - mn) for v in blk)
        m = mn
        out.append((m, l))
    return out


def softmax_two_pass(x):
    """Safe softmax by definition: max, then sum, then divide."""
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def state(s: np.ndarray, v: np.ndarray):
    """Partial state (m, l, o) of one key set: s [n] scores, v [n, hd] values."""
    m = float(np.max(s))
    p = np.exp(s - m)
    return m, float(p.sum()), p @ v


def merge(a, b):
    """(m, l, o) of the union of two disjoint key sets."""
    ma, la, oa = a
    mb, lb, ob = b
    m = max(ma, mb)
    ea = math.exp(ma - m) if ma != -math.inf else 0.0
    eb = math.exp(mb - m) if mb != -math.inf else 0.0
    return m, la * ea + lb * eb, oa * ea + ob * eb


def finish(st):
    m, l, o = st
    return o / l, m + math.log(l)


def tiled_forward(q, k, v, scale: float, causal: bool, br: int, bc: int, rescale: bool = True,
                  dtype=np.float64):
    """One head, q/k/v [T, hd]; query tiles of br rows, key blocks of bc rows.

    Returns (O [T, hd], L [T]).  Rows past T in a tile and keys past T in a
    block are excluded; in causal mode key j is visible to row i iff j <= i.
    ``dtype=np.float32`` runs every step in float32 (the tiled float32 output
    the lesson's checker control must accept).
    """
    q = np.asarray(q, dtype)
    k = np.asarray(k, dtype)
    v = np.asarray(v, dtype)
    scale = dtype(scale)
    T, hd = q.shape
    O = np.zeros((T, hd), dtype)
    L = np.zeros(T, dtype)
    for i0 in range(0, T, br):
        rows = range(i0, min(i0 + br, T))
        last = rows[-1]
        m = np.full(len(rows), -np.inf, dtype)
        l = np.zeros(len(rows), dtype)
        o = np.zeros((len(rows), hd), dtype)
        for j0 in range(0, T, bc):
            if causal and j0 > last:
                break  # every later block is wholly above the diagonal
            cols = np.arange(j0, min(j0 + bc, T))
            s = scale * (q[i0:last + 1] @ k[cols].T)
            if causal:
                s = np.where(cols[None, :] > np.arange(i0, last + 1)[:, None], -np.inf, s)
            mb = s.max(axis=1)
            mn = np.maximum(m, mb)
            if rescale:
                alpha = np.where(m == -np.inf, dtype(0), np.exp(m - mn)).astype(dtype)
            else:
                alpha = np.ones_like(m)
            p = np.where(np.isneginf(s), dtype(0), np.exp(s - np.where(np.isneginf(mn), dtype(0), mn)[:, None]))
            p = p.astype(dtype)
            l = l * alpha + p.sum(axis=1)
            o = o * alpha[:, None] + p @ v[cols]
            m = mn
        O[i0:last + 1] = o / l[:, None]
        L[i0:last + 1] = m + np.log(l)
    return O, L
