"""Tiled online-softmax attention in float64: a second CPU implementation.

TEST INFRASTRUCTURE ONLY (same rules as ``oracle.attention``).  It exists to pin
the claim the pages make about the method, namely that tiling plus an online
softmax reaches *exactly* the result of the plain two-pass definition, so tests
compare it with ``oracle.attention`` in float64.  It is never compared with the GPU
path directly.

Steps, in the order the pages give them:

* "LLM interview question bank" ch.029, question #36, section 3 (Tiling + Online
  Softmax): for each Q tile of Br rows, initialise the running statistics (m, l);
  for each K/V tile of Bc rows, form the score tile, update m and l, add the tile's
  contribution to the output accumulator and discard the score tile; write the
  output tile once at the end.
* Stanford lecture summary (youtublog.net), section "推导 FlashAttention 的在线
  softmax": the output is numerator / denominator; both are rescaled by
  exp(m_old - m_new) whenever the running maximum grows, which avoids overflow of
  exp; very small terms may underflow.
"""
from __future__ import annotations

import math

import numpy as np


def online_softmax_states(x, v):
    """Scalar recurrence over one row: returns [(m, l, num)] after each element.

    x are scores and v scalar values; the final output is num / l.  The running
    maximum m starts at -inf; each new element rescales the old numerator and
    denominator by exp(m_old - m_new) before adding its own exp(x - m_new).
    """
    m, l, num = -math.inf, 0.0, 0.0
    states = []
    for xi, vi in zip(x, v):
        m_new = max(m, xi)
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        e = math.exp(xi - m_new)
        l = alpha * l + e
        num = alpha * num + e * vi
        m = m_new
        states.append((m, l, num))
    return states


def head_forward_tiled(q, k, v, causal: bool, scale: float, br: int, bc: int):
    """One head, tiled with Br query rows and Bc key rows: (O [N, d], LSE [N])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(n, i0 + br))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, v.shape[1]))
        for j0 in range(0, n, bc):
            cols = np.arange(j0, min(n, j0 + bc))
            s = scale * (q[rows] @ k[cols].T)
            if causal:
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            # rows whose visible keys all lie in later tiles keep m = -inf
            live = np.isfinite(m_new)
            safe = np.where(live, m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
            p = np.exp(s - safe[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse
