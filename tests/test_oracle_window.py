"""Pins of the oracle's sliding-window mask: query i sees key j only if |i - j| <=
window (and j <= i when causal).

Pinned against closed forms (window 0 and 1), brute-force scalar loops, an
independent library routine with an explicit band mask, central finite differences
of the gradients, and planted off-by-one mistakes.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as A
from oracle import attention_backward, attention_forward, head_backward, head_forward


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [True, False])
def test_window_zero_sees_only_itself(causal):
    # |i - j| <= 0: every row's softmax has one term, so O_i = V_i and LSE_i = scale q_i.k_i
    n, d = 9, 4
    q, k, v = rand((n, d), 1), rand((n, d), 2), rand((n, d), 3)
    o, lse = head_forward(q, k, v, causal, 0.7, window=0)
    assert np.abs(o - v).max() <= 1e-15
    assert np.abs(lse - 0.7 * (q * k).sum(axis=1)).max() <= 1e-14


def test_causal_window_one_is_a_two_term_softmax():
    # row i >= 1 sees keys i-1 and i: O_i = sigmoid(s_ii - s_i,i-1) V_i + (1 - .) V_{i-1}
    n, d, sc = 7, 3, 0.9
    q, k, v = rand((n, d), 4), rand((n, d), 5), rand((n, d), 6)
    o, lse = head_forward(q, k, v, True, sc, window=1)
    for i in range(1, n):
        a, b = sc * q[i] @ k[i - 1], sc * q[i] @ k[i]
        w = 1.0 / (1.0 + math.exp(a - b))
        assert np.abs(o[i] - (w * v[i] + (1 - w) * v[i - 1])).max() <= 1e-14
        assert lse[i] == pytest.approx(np.logaddexp(a, b), abs=1e-14)
    assert np.abs(o[0] - v[0]).max() <= 1e-15


def test_window_wider_than_the_sequence_is_no_window():
    n, d = 12, 5
    q, k, v, do = rand((n, d), 7), rand((n, d), 8), rand((n, d), 9), rand((n, d), 10)
    for causal in (True, False):
        o1, l1 = head_forward(q, k, v, causal, 0.4, window=n - 1)
        o2, l2 = head_forward(q, k, v, causal, 0.4)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        g1 = head_backward(q, k, v, do, causal, 0.4, window=n + 5)
        g2 = head_backward(q, k, v, do, causal, 0.4)
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)


def _brute_window(q, k, v, do, causal, window, scale):
    """Scalar loops with math.fsum; the band written out independently."""
    n, d = len(q), len(q[0])
    vis = [[abs(i - j) <= window and (j <= i or not causal) for j in range(n)] for i in range(n)]
    s = [[scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in range(n)] for i in range(n)]
    p, o, lse = [], [], []
    for i in range(n):
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


@pytest.mark.parametrize("window", [0, 1, 2, 5])
@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_scalar_loops(window, causal):
    n, d = 8, 3
    q, k, v, do = rand((n, d), 20 + window), rand((n, d), 30), rand((n, d), 40), rand((n, d), 50)
    o, lse = head_forward(q, k, v, causal, 0.8, window=window)
    dq, dk, dv = head_backward(q, k, v, do, causal, 0.8, window=window)
    ref = _brute_window(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, window, 0.8)
    for a, b in zip((o, lse, dq, dk, dv), ref):
        assert np.abs(a - np.array(b)).max() <= 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_cpu_float64_sdpa_with_band_mask(causal):
    b, hq, hkv, n, d, scale, w = 2, 4, 2, 40, 8, 0.3, 6
    q, k, v, do = rand((b, hq, n, d), 60), rand((b, hkv, n, d), 61), rand((b, hkv, n, d), 62), \
        rand((b, hq, n, d), 63)
    i, j = torch.arange(n)[:, None], torch.arange(n)[None, :]
    mask = (i - j).abs() <= w
    if causal:
        mask = mask & (j <= i)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    g = hq // hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=mask, scale=scale)
    out.backward(torch.tensor(do))
    o, _ = attention_forward(q, k, v, causal, scale, window=w)
    dq, dk, dv = attention_backward(q, k, v, do, causal, scale, window=w)
    assert np.abs(o - out.detach().numpy()).max() < 1e-12
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-12


def test_window_gradients_by_central_differences():
    n, d, w, sc, h = 6, 3, 2, 0.6, 1e-6
    q, k, v, do = rand((n, d), 70), rand((n, d), 71), rand((n, d), 72), rand((n, d), 73)
    loss = lambda q_, k_, v_: float((head_forward(q_, k_, v_, True, sc, window=w)[0] * do).sum())
    dq, dk, dv = head_backward(q, k, v, do, True, sc, window=w)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if x is y else y for y in (q, k, v)]
            args_m = [xm if x is y else y for y in (q, k, v)]
            num = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert num == pytest.approx(g[idx], rel=1e-6, abs=1e-8)


def _scores_window_off_by_one(q_rows, k, rows, causal, scale, window=-1, block_mask=None):
    s = scale * (q_rows @ k.T)
    cols = np.arange(k.shape[0])
    if causal:
        s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
    if window >= 0:
        s = np.where(np.abs(cols[None, :] - rows[:, None]) < window, s, -np.inf)
    return s


def _scores_window_one_sided(q_rows, k, rows, causal, scale, window=-1, block_mask=None):
    s = scale * (q_rows @ k.T)
    cols = np.arange(k.shape[0])
    if causal:
        s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
    if window >= 0:
        s = np.where(rows[:, None] - cols[None, :] <= window, s, -np.inf)
    return s


@pytest.mark.parametrize("wrong", [_scores_window_off_by_one, _scores_window_one_sided])
def test_planted_window_mistakes_are_caught(monkeypatch, wrong):
    monkeypatch.setattr(A, "_scores", wrong)
    n, d = 8, 3
    q, k, v, do = rand((n, d), 80), rand((n, d), 81), rand((n, d), 82), rand((n, d), 83)
    caught = False
    for causal in (True, False):
        with np.errstate(all="ignore"):
            o, _ = A.head_forward(q, k, v, causal, 0.8, window=2)
        ref = _brute_window(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, 2, 0.8)
        caught |= bool(np.isnan(o).any() or np.abs(o - np.array(ref[0])).max() > 1e-9)
    assert caught
