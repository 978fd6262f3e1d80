"""Pins of the oracle's decode form (Nq new queries against a cache of Nk keys).

The queries are the last Nq tokens of a sequence whose Nk keys and values, their own
included, are cached; query i sits at position Nk - Nq + i.  Each test pins that
reading to something other than ``decode_forward`` itself: the already pinned
full-sequence oracle, brute-force scalar loops, an independent library routine,
a closed form, and the merge of two key ranges by their log-sum-exp.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as A
from oracle import attention_forward, decode_forward


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("nq", [1, 3, 17])
def test_decode_rows_are_the_tail_of_the_full_sequence(causal, nq):
    # Decoding the last nq tokens against the whole cache gives the last nq rows of
    # the full-sequence result (whose causal mask is pinned by the hand example,
    # brute force and the library routine in test_oracle.py).
    b, hq, hkv, n, d = 2, 6, 2, 40, 8
    q, k, v = rand((b, hq, n, d), 1), rand((b, hkv, n, d), 2), rand((b, hkv, n, d), 3)
    o_full, lse_full = attention_forward(q, k, v, causal, 0.4)
    o, lse = decode_forward(q[:, :, n - nq:], k, v, causal, 0.4)
    assert np.abs(o - o_full[:, :, n - nq:]).max() <= 1e-13
    assert np.abs(lse - lse_full[:, :, n - nq:]).max() <= 1e-13


def test_single_new_token_sees_the_whole_cache():
    b, hq, hkv, nk, d = 1, 4, 1, 23, 5
    q, k, v = rand((b, hq, 1, d), 4), rand((b, hkv, nk, d), 5), rand((b, hkv, nk, d), 6)
    oc, lc = decode_forward(q, k, v, True, 0.7)
    on, ln = decode_forward(q, k, v, False, 0.7)
    assert np.array_equal(oc, on) and np.array_equal(lc, ln)


def test_zero_queries_average_the_visible_values():
    # Q = 0: every visible key has the same score, so O is the mean of the visible
    # values and LSE = ln(number of visible keys).
    nq, nk, d = 4, 11, 3
    v = rand((1, 1, nk, d), 7)
    o, lse = decode_forward(np.zeros((1, 1, nq, d)), rand((1, 1, nk, d), 8), v, True, 1.0)
    for i in range(nq):
        seen = nk - nq + i + 1
        assert np.abs(o[0, 0, i] - v[0, 0, :seen].mean(axis=0)).max() <= 1e-15
        assert lse[0, 0, i] == pytest.approx(math.log(seen), abs=1e-15)


def _brute_decode(q, k, v, causal, scale):
    """Scalar loops with math.fsum; positions written out independently."""
    nq, nk, d = len(q), len(k), len(q[0])
    o, lse = [], []
    for i in range(nq):
        pos = nk - nq + i
        vis = [j for j in range(nk) if j <= pos or not causal]
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in vis}
        mx = max(s.values())
        z = math.fsum(math.exp(s[j] - mx) for j in vis)
        o.append([math.fsum(math.exp(s[j] - mx) / z * v[j][t] for j in vis) for t in range(d)])
        lse.append(mx + math.log(z))
    return o, lse


@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 7), (3, 8), (5, 5), (2, 9)])
@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_scalar_loops(nq, nk, causal):
    d = 3
    q, k, v = rand((nq, d), 10 + nk), rand((nk, d), 20 + nk), rand((nk, d), 30 + nk)
    o, lse = decode_forward(q[None, None], k[None, None], v[None, None], causal, 0.9)
    bo, bl = _brute_decode(q.tolist(), k.tolist(), v.tolist(), causal, 0.9)
    assert np.abs(o[0, 0] - np.array(bo)).max() <= 1e-13
    assert np.abs(lse[0, 0] - np.array(bl)).max() <= 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_cpu_float64_sdpa_with_explicit_mask(causal):
    b, hq, hkv, nq, nk, d, scale = 2, 6, 2, 5, 29, 16, 0.25
    q, k, v = rand((b, hq, nq, d), 40), rand((b, hkv, nk, d), 41), rand((b, hkv, nk, d), 42)
    g = hq // hkv
    mask = None
    if causal:   # query i at position nk - nq + i sees keys j <= that position
        mask = torch.arange(nk)[None, :] <= (nk - nq + torch.arange(nq))[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k).repeat_interleave(g, dim=1),
        torch.tensor(v).repeat_interleave(g, dim=1), attn_mask=mask, scale=scale)
    o, _ = decode_forward(q, k, v, causal, scale)
    assert np.abs(o - out.numpy()).max() < 1e-12


def test_two_key_ranges_merge_by_log_sum_exp():
    # Softmax over a union of key ranges: each range's (O, LSE) combine with weights
    # exp(LSE_s - LSE), LSE = log(sum_s exp(LSE_s)) -- the rescaling of the online
    # softmax applied to whole partial results.
    b, hq, hkv, nq, nk, d, cut = 1, 3, 1, 4, 30, 6, 13
    q, k, v = rand((b, hq, nq, d), 50), rand((b, hkv, nk, d), 51), rand((b, hkv, nk, d), 52)
    o, lse = decode_forward(q, k, v, False, 0.5)
    o1, l1 = decode_forward(q, k[:, :, :cut], v[:, :, :cut], False, 0.5)
    o2, l2 = decode_forward(q, k[:, :, cut:], v[:, :, cut:], False, 0.5)
    lm = np.logaddexp(l1, l2)
    om = np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2
    assert np.abs(lm - lse).max() <= 1e-13
    assert np.abs(om - o).max() <= 1e-13


def test_top_left_alignment_is_caught(monkeypatch):
    # A plausible mistake, the full-sequence mask j <= i applied to the new queries,
    # must fail the tail-of-the-sequence pin.
    monkeypatch.setattr(A, "_query_offset", lambda nq, nk: 0)
    b, hq, hkv, n, d, nq = 1, 2, 1, 12, 4, 3
    q, k, v = rand((b, hq, n, d), 60), rand((b, hkv, n, d), 61), rand((b, hkv, n, d), 62)
    o_full, _ = attention_forward(q, k, v, True, 0.6)
    o, _ = decode_forward(q[:, :, n - nq:], k, v, True, 0.6)
    assert np.abs(o - o_full[:, :, n - nq:]).max() > 1e-3


def test_shape_checks():
    with pytest.raises(ValueError):
        decode_forward(np.zeros((1, 3, 1, 4)), np.zeros((1, 2, 5, 4)), np.zeros((1, 2, 5, 4)), True, 1.0)
    with pytest.raises(ValueError):
        decode_forward(np.zeros((1, 2, 1, 4)), np.zeros((1, 1, 5, 4)), np.zeros((1, 1, 6, 4)), True, 1.0)
