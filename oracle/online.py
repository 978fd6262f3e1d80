"""Online-softmax attention in float64 built from per-tile partial states: a second
CPU implementation.

TEST INFRASTRUCTURE ONLY (same rules as ``oracle.attention``).  It exists to pin
the claim the pages make about the method, namely that cutting the keys into tiles
and combining the tiles' softmax statistics reaches *exactly* the result of the
plain two-pass definition, so tests compare it with ``oracle.attention`` in
float64.  It is never compared with the GPU path directly.

It is derived from the mathematics rather than from any printed loop.  For one
query row and a set T of keys with scores s_j, the partial state is

    m_T = max_{j in T} s_j,   l_T = sum_{j in T} exp(s_j - m_T),
    a_T = sum_{j in T} exp(s_j - m_T) v_j.

Two states over disjoint key sets combine into the state of their union:

    m = max(m_A, m_B),  l = l_A e^(m_A - m) + l_B e^(m_B - m),
    a = a_A e^(m_A - m) + a_B e^(m_B - m),

an associative and commutative operation (exp(m_A - m) rescales A's terms from its
own reference m_A to the common one).  The output of the whole row is a / l and
its log-sum-exp m + log l.  The sources state this rescaling in words:

* Stanford lecture summary (youtublog.net), section "推导 FlashAttention 的在线
  softmax": an output row is a numerator over a denominator, and both are rescaled
  by exp(m_old - m_new) when the reference maximum changes, which keeps exp from
  overflowing (tiny terms may underflow).
* "LLM interview question bank" ch.029 (ricardokevins.github.io), question #36,
  section 3 (Tiling + Online Softmax): the score tile of a K/V tile is used on chip
  and dropped; only the running statistics and the output accumulator are kept.

Because the merge is associative, the tiles are combined here in a seeded random
tree order (not left to right), which is a stronger check than replaying the
sequential loop: any mistake in the rescaling shows up for some order.
"""
from __future__ import annotations

import math

import numpy as np


def online_softmax_states(x, v):
    """Scalar recurrence over one row: returns [(m, l, num)] after each element.

    x are scores and v scalar values; the final output is num / l.  The running
    maximum m starts at -inf; each new element rescales the old numerator and
    denominator by exp(m_old - m_new) before adding its own exp(x - m_new).  This is
    the merge below applied to one-element key sets, left to right.
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


def tile_state(s, v):
    """Partial state (m, l, a) of every row over one key tile.

    s: [rows, keys] scores of the tile (-inf where a key is not visible);
    v: [keys, d] the tile's values.  A row that sees no key of the tile gets
    m = -inf, l = 0, a = 0 (the identity of the merge).
    """
    m = s.max(axis=1)
    live = np.isfinite(m)
    e = np.exp(s - np.where(live, m, 0.0)[:, None])   # exp(-inf) = 0 for hidden keys
    e = np.where(live[:, None], e, 0.0)
    return m, e.sum(axis=1), e @ v


def merge_states(a, b):
    """State of the union of two disjoint key sets (associative, commutative)."""
    ma, la, aa = a
    mb, lb, ab = b
    m = np.maximum(ma, mb)
    safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(ma), np.exp(ma - safe), 0.0)
    wb = np.where(np.isfinite(mb), np.exp(mb - safe), 0.0)
    return m, la * wa + lb * wb, aa * wa[:, None] + ab * wb[:, None]


def head_forward_merged(q, k, v, causal: bool, scale: float, bc: int, seed: int = 0):
    """One head, keys cut into tiles of ``bc``: (O [N, d], LSE [N]).

    Every tile's state is formed on its own, then the states are merged pairwise in
    a tree whose leaf order is a seeded permutation of the tiles.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n)
    states = []
    for j0 in range(0, k.shape[0], bc):
        cols = np.arange(j0, min(k.shape[0], j0 + bc))
        s = scale * (q @ k[cols].T)
        if causal:
            s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
        states.append(tile_state(s, v[cols]))
    order = np.random.default_rng(seed).permutation(len(states))
    level = [states[i] for i in order]
    while len(level) > 1:
        nxt = [merge_states(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    m, l, acc = level[0]
    return acc / l[:, None], m + np.log(l)
