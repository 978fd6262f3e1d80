"""Planted mistakes in the CPU oracle must be caught by the pins.

Each case patches one plausible mistake into ``oracle.attention`` (on the CPU only)
and checks that an independent pin (hand example, brute force, finite differences,
grouped-query equivalence) no longer holds.  Nothing here touches the GPU path.
"""
import math

import numpy as np
import pytest

import oracle.attention as A
from tests.test_oracle import _brute_head, _golden_attention, rand


def _pins_hold() -> bool:
    """A compact run of the forward/backward pins; False as soon as one fails."""
    g = _golden_attention()
    q = np.ones((3, 1))
    k = np.array([[0.0], [math.log(2)], [math.log(3)]])
    v = np.array([[1.0], [2.0], [3.0]])
    o, lse = A.head_forward(q, k, v, True, 1.0)
    if any(abs(o[i, 0] - g[("O_causal", i)]) > 1e-12 or abs(lse[i] - g[("LSE_causal", i)]) > 1e-12
           for i in range(3)):
        return False
    dq, dk, dv = A.head_backward(q, k, v, np.ones((3, 1)), True, 1.0)
    if any(abs(dk[i, 0] - g[("dK_causal", i)]) > 1e-12 or abs(dv[i, 0] - g[("dV_causal", i)]) > 1e-12
           or abs(dq[i, 0] - g[("dQ_causal", i)]) > 1e-12 for i in range(3)):
        return False
    for causal in (True, False):
        n, d = 6, 3
        qq, kk, vv, dd = rand((n, d), 1), rand((n, d), 2), rand((n, d), 3), rand((n, d), 4)
        bo, bl, bdq, bdk, bdv = _brute_head(qq.tolist(), kk.tolist(), vv.tolist(), dd.tolist(), causal, 0.7)
        o, lse = A.head_forward(qq, kk, vv, causal, 0.7)
        dq, dk, dv = A.head_backward(qq, kk, vv, dd, causal, 0.7)
        for a, b in ((o, bo), (lse, bl), (dq, bdq), (dk, bdk), (dv, bdv)):
            if np.abs(a - np.array(b)).max() > 1e-12:
                return False
    b, hq, hkv, n, d = 1, 4, 2, 5, 3
    qq, kk, vv = rand((b, hq, n, d), 5), rand((b, hkv, n, d), 6), rand((b, hkv, n, d), 7)
    o, _ = A.attention_forward(qq, kk, vv, False, 0.5)
    o2, _ = A.attention_forward(qq, np.repeat(kk, 2, axis=1), np.repeat(vv, 2, axis=1), False, 0.5)
    return np.abs(o - o2).max() < 1e-12


def test_unpatched_oracle_passes():
    assert _pins_hold()


def _scores_no_scale(q_rows, k, rows, causal, scale, window=-1, block_mask=None):
    s = q_rows @ k.T
    if causal:
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
    return s


def _scores_strict_mask(q_rows, k, rows, causal, scale, window=-1, block_mask=None):
    s = scale * (q_rows @ k.T)
    if causal:
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] < rows[:, None], s, -np.inf)
    return s


def _scores_upper_mask(q_rows, k, rows, causal, scale, window=-1, block_mask=None):
    s = scale * (q_rows @ k.T)
    if causal:
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] >= rows[:, None], s, -np.inf)
    return s


def _bwd_wrong_sign(q, k, v, do, causal, scale, window=-1, block_mask=None):
    dq, dk, dv = _orig_bwd(q, k, v, do, causal, scale)
    return -dq, -dk, dv


def _bwd_no_d_term(q, k, v, do, causal, scale, window=-1, block_mask=None):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    rows = np.arange(q.shape[0])
    p = A.head_probs(q, k, causal, scale)
    ds = p * (do @ v.T)                      # dropped "- D"
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


def _bwd_transposed_dv(q, k, v, do, causal, scale, window=-1, block_mask=None):
    dq, dk, dv = _orig_bwd(q, k, v, do, causal, scale)
    p = A.head_probs(q, k, causal, scale)
    return dq, dk, p @ np.asarray(do, dtype=np.float64)   # P dO instead of P^T dO


def _group_interleaved(hq, hq_total, hkv_total):
    return hq % hkv_total


_orig_bwd = A.head_backward


@pytest.mark.parametrize("target,replacement", [
    ("_scores", _scores_no_scale),
    ("_scores", _scores_strict_mask),
    ("_scores", _scores_upper_mask),
    ("head_backward", _bwd_wrong_sign),
    ("head_backward", _bwd_no_d_term),
    ("head_backward", _bwd_transposed_dv),
    ("_group", _group_interleaved),
])
def test_planted_mistake_is_caught(monkeypatch, target, replacement):
    monkeypatch.setattr(A, target, replacement)
    with np.errstate(all="ignore"):
        try:
            held = _pins_hold()
        except (ValueError, FloatingPointError, ZeroDivisionError):
            held = False
    assert not held
