"""Pins of the oracle's block-sparse layout: query i sees key j only if
block_mask[i // BLOCK][j // BLOCK] is set (and j <= i when causal).

Pinned by: an all-ones layout and a lower-triangular layout under the causal rule
equal the dense calls; a block-diagonal layout equals independent attention on each
block (forward and gradients); brute-force scalar loops and central finite
differences at a small block size; torch's float64 SDPA with the expanded mask;
rows that see nothing (O = 0, LSE = -inf, no gradient); a planted transposed layout.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as A
from oracle import attention_backward, attention_forward, head_backward, head_forward


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_ones_and_causal_triangle_equal_the_dense_calls():
    n, d = 150, 8
    q, k, v, do = rand((n, d), 1), rand((n, d), 2), rand((n, d), 3), rand((n, d), 4)
    nb = -(-n // A.BLOCK)
    ones, tri = np.ones((nb, nb), bool), np.tril(np.ones((nb, nb), bool))
    for causal, bm in ((False, ones), (True, ones), (True, tri)):
        o1, l1 = head_forward(q, k, v, causal, 0.3, block_mask=bm)
        o2, l2 = head_forward(q, k, v, causal, 0.3)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        for a, b in zip(head_backward(q, k, v, do, causal, 0.3, block_mask=bm), head_backward(q, k, v, do, causal, 0.3)):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [True, False])
def test_block_diagonal_layout_is_attention_within_each_block(causal):
    n, d, B = 200, 6, A.BLOCK
    q, k, v, do = rand((n, d), 5), rand((n, d), 6), rand((n, d), 7), rand((n, d), 8)
    nb = -(-n // B)
    o, lse = head_forward(q, k, v, causal, 0.4, block_mask=np.eye(nb, dtype=bool))
    dq, dk, dv = head_backward(q, k, v, do, causal, 0.4, block_mask=np.eye(nb, dtype=bool))
    for b0 in range(0, n, B):
        sl = slice(b0, min(n, b0 + B))
        ob, lb = head_forward(q[sl], k[sl], v[sl], causal, 0.4)
        gb = head_backward(q[sl], k[sl], v[sl], do[sl], causal, 0.4)
        assert np.abs(o[sl] - ob).max() <= 1e-14 and np.abs(lse[sl] - lb).max() <= 1e-14
        for a, g in zip((dq, dk, dv), gb):
            assert np.abs(a[sl] - g).max() <= 1e-14


def _brute_blocks(q, k, v, do, causal, bm, bs, scale):
    """Scalar loops with math.fsum; the layout test written out independently."""
    n, d = len(q), len(q[0])
    vis = [[bool(bm[i // bs][j // bs]) and (j <= i or not causal) for j in range(n)] for i in range(n)]
    s = [[scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in range(n)] for i in range(n)]
    p, o, lse = [], [], []
    for i in range(n):
        if not any(vis[i]):
            p.append([0.0] * n)
            o.append([0.0] * d)
            lse.append(-math.inf)
            continue
        mx = max(s[i][j] for j in range(n) if vis[i][j])
        z = math.fsum(math.exp(s[i][j] - mx) for j in range(n) if vis[i][j])
        row = [math.exp(s[i][j] - mx) / z if vis[i][j] else 0.0 for j in range(n)]
        p.append(row)
        o.append([math.fsum(row[j] * v[j][t] for j in range(n)) for t in range(d)])
        lse.append(mx + math.log(z))
    dpm = [[math.fsum(do[i][t] * v[j][t] for t in range(d)) for j in range(n)] for i in range(n)]
    dd = [math.fsum(p[i][j] * dpm[i][j] for j in range(n)) for i in range(n)]
    ds = [[p[i][j] * (dpm[i][j] - dd[i]) for j in range(n)] for i in range(n)]
    dq = [[scale * math.fsum(ds[i][j] * k[j][t] for j in range(n)) for t in range(d)] for i in range(n)]
    dk = [[scale * math.fsum(ds[i][j] * q[i][t] for i in range(n)) for t in range(d)] for j in range(n)]
    dv = [[math.fsum(p[i][j] * do[i][t] for i in range(n)) for t in range(d)] for j in range(n)]
    return o, lse, dq, dk, dv


LAYOUT = np.array([[1, 1, 0, 0], [0, 1, 0, 1], [1, 0, 1, 0], [0, 1, 1, 1]], dtype=bool)   # not symmetric


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_scalar_loops_small_blocks(monkeypatch, causal):
    monkeypatch.setattr(A, "BLOCK", 2)
    n, d = 8, 3
    q, k, v, do = rand((n, d), 10), rand((n, d), 11), rand((n, d), 12), rand((n, d), 13)
    o, lse = head_forward(q, k, v, causal, 0.8, block_mask=LAYOUT)
    g = head_backward(q, k, v, do, causal, 0.8, block_mask=LAYOUT)
    ref = _brute_blocks(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, LAYOUT, 2, 0.8)
    assert np.abs(o - np.array(ref[0])).max() <= 1e-13
    fin = np.isfinite(ref[1])
    assert np.abs(lse[fin] - np.array(ref[1])[fin]).max() <= 1e-13 and np.isneginf(lse[~fin]).all()
    for a, b in zip(g, ref[2:]):
        assert np.abs(a - np.array(b)).max() <= 1e-13


def test_rows_that_see_nothing():
    # under the causal rule a query block whose only set blocks lie after it sees no key
    n, d = 128, 4
    bm = np.array([[0, 1], [1, 1]], dtype=bool)
    q, k, v, do = rand((n, d), 14), rand((n, d), 15), rand((n, d), 16), rand((n, d), 17)
    o, lse = head_forward(q, k, v, True, 0.5, block_mask=bm)
    dq, dk, dv = head_backward(q, k, v, do, True, 0.5, block_mask=bm)
    assert (o[:64] == 0).all() and np.isneginf(lse[:64]).all() and (dq[:64] == 0).all()
    assert np.isfinite(lse[64:]).all()


@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_cpu_float64_sdpa_with_the_expanded_layout(causal):
    b, hq, hkv, n, d, scale = 1, 4, 2, 3 * A.BLOCK - 10, 8, 0.3
    bm = np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=bool)   # every row sees its own block
    q, k, v, do = rand((b, hq, n, d), 20), rand((b, hkv, n, d), 21), rand((b, hkv, n, d), 22), rand((b, hq, n, d), 23)
    idx = np.arange(n) // A.BLOCK
    mask = torch.tensor(bm[idx[:, None], idx[None, :]])
    if causal:
        mask = mask & torch.tril(torch.ones(n, n, dtype=torch.bool))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    g = hq // hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=mask, scale=scale)
    out.backward(torch.tensor(do))
    o, _ = attention_forward(q, k, v, causal, scale, block_mask=bm)
    dq, dk, dv = attention_backward(q, k, v, do, causal, scale, block_mask=bm)
    assert np.abs(o - out.detach().numpy()).max() < 1e-12
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-12


def test_gradients_by_central_differences_small_blocks(monkeypatch):
    monkeypatch.setattr(A, "BLOCK", 2)
    n, d, sc, h = 8, 2, 0.6, 1e-6
    q, k, v, do = rand((n, d), 30), rand((n, d), 31), rand((n, d), 32), rand((n, d), 33)
    loss = lambda q_, k_, v_: float((head_forward(q_, k_, v_, False, sc, block_mask=LAYOUT)[0] * do).sum())
    dq, dk, dv = head_backward(q, k, v, do, False, sc, block_mask=LAYOUT)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num = (loss(*[xp if x is y else y for y in (q, k, v)]) - loss(*[xm if x is y else y for y in (q, k, v)])) / (2 * h)
            assert num == pytest.approx(g[idx], rel=1e-6, abs=1e-8)


def test_planted_transposed_layout_is_caught(monkeypatch):
    assert not np.array_equal(LAYOUT, LAYOUT.T)
    def wrong(q_rows, k, rows, causal, scale, window=-1, block_mask=None):
        s = scale * (q_rows @ k.T)
        cols = np.arange(k.shape[0])
        bm = np.asarray(block_mask, dtype=bool)
        return np.where(bm[cols[None, :] // A.BLOCK, rows[:, None] // A.BLOCK], s, -np.inf)
    monkeypatch.setattr(A, "BLOCK", 2)
    n, d = 8, 3
    q, k, v, do = rand((n, d), 40), rand((n, d), 41), rand((n, d), 42), rand((n, d), 43)
    ref = _brute_blocks(q.tolist(), k.tolist(), v.tolist(), do.tolist(), False, LAYOUT, 2, 0.8)
    monkeypatch.setattr(A, "_scores", wrong)
    with np.errstate(all="ignore"):
        o, _ = A.head_forward(q, k, v, False, 0.8, block_mask=LAYOUT)
    assert np.abs(o - np.array(ref[0])).max() > 1e-6
