"""Pins of the CPU float64 oracle against facts that do not come from the oracle.

Each test names the fact it pins and where it comes from: a worked example with
hand-derived values (tests/golden/), a closed form, an invariant of the softmax,
brute force on tiny inputs, finite differences, or an independent library routine.
"""
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_forward, head_backward, head_forward,
                    head_forward_merged, head_probs, merge_states, online_softmax_states,
                    tile_state)

GOLDEN = Path(__file__).parent / "golden"


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------ P1: worked example

def test_three_element_online_example_matches_hand_values():
    rows = [ln.split() for ln in (GOLDEN / "online_softmax_three_elements.txt").read_text().splitlines()
            if ln and not ln.startswith("#") and not ln.startswith("step")]
    steps = [r for r in rows if r[0] != "output"]
    out = [r for r in rows if r[0] == "output"][0]
    x = [0.0, math.log(2.0), math.log(3.0)]
    v = [1.0, 2.0, 3.0]
    states = online_softmax_states(x, v)
    for (m, l, num), r in zip(states, steps):
        _, marg, ln_, ld, nn, nd = r
        assert m == pytest.approx(math.log(int(marg)), abs=1e-15)
        assert l == pytest.approx(int(ln_) / int(ld), rel=1e-15)
        assert num == pytest.approx(int(nn) / int(nd), rel=1e-15)
    m, l, num = states[-1]
    assert num / l == pytest.approx(int(out[1]) / int(out[2]), rel=1e-15)
    # the plain definition on the same numbers
    e = np.exp(np.array(x))
    assert float(e @ np.array(v) / e.sum()) == pytest.approx(7 / 3, rel=1e-15)


def test_three_element_example_survives_overflow():
    # Shifting every score by 1000 overflows a naive exp in float64 but not the
    # running-max recurrence (the lecture's reason for subtracting the running max).
    x = [1000.0, 1000.0 + math.log(2.0), 1000.0 + math.log(3.0)]
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.array(x))).all()
    m, l, num = online_softmax_states(x, [1.0, 2.0, 3.0])[-1]
    assert num / l == pytest.approx(7 / 3, rel=1e-14)


# ------------------------------------------------------------------ hand-derived attention

def _golden_attention():
    vals = {}
    for ln in (GOLDEN / "attention_hand_example.txt").read_text().splitlines():
        if not ln or ln.startswith("#"):
            continue
        name, i, num, den, c2, c3, c6 = ln.split()
        vals[(name, int(i))] = (float(Fraction(int(num), int(den))) + float(c2) * math.log(2)
                                + float(c3) * math.log(3) + float(c6) * math.log(6))
    return vals


@pytest.mark.parametrize("causal", [True, False])
def test_hand_example_forward(causal):
    g = _golden_attention()
    q = np.ones((3, 1))
    k = np.array([[0.0], [math.log(2)], [math.log(3)]])
    v = np.array([[1.0], [2.0], [3.0]])
    o, lse = head_forward(q, k, v, causal, 1.0)
    tag = "causal" if causal else "full"
    for i in range(3):
        assert o[i, 0] == pytest.approx(g[(f"O_{tag}", i)], abs=1e-14)
        assert lse[i] == pytest.approx(g[(f"LSE_{tag}", i)], abs=1e-14)


def test_hand_example_backward():
    g = _golden_attention()
    q = np.ones((3, 1))
    k = np.array([[0.0], [math.log(2)], [math.log(3)]])
    v = np.array([[1.0], [2.0], [3.0]])
    dq, dk, dv = head_backward(q, k, v, np.ones((3, 1)), True, 1.0)
    for i in range(3):
        assert dq[i, 0] == pytest.approx(g[("dQ_causal", i)], abs=1e-14)
        assert dk[i, 0] == pytest.approx(g[("dK_causal", i)], abs=1e-14)
        assert dv[i, 0] == pytest.approx(g[("dV_causal", i)], abs=1e-14)


# ------------------------------------------------------------------ P2, P3: softmax invariants

def test_rows_of_p_sum_to_one():
    for causal in (True, False):
        p = head_probs(rand((37, 8), 1), rand((37, 8), 2), causal, 0.7)
        assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-14
        assert (p >= 0).all()
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


def test_shift_invariance():
    # Adding c_i to every score of row i leaves P and O unchanged and shifts LSE by c_i.
    # With d+1 features, appending q_i,d = c_i/scale and k_j,d = 1 adds exactly c_i.
    n, d, scale = 29, 6, 0.5
    q, k, v = rand((n, d), 3), rand((n, d), 4), rand((n, d), 5)
    c = rand(n, 6, 10.0)
    q2 = np.concatenate([q, (c / scale)[:, None]], axis=1)
    k2 = np.concatenate([k, np.ones((n, 1))], axis=1)
    for causal in (True, False):
        o1, l1 = head_forward(q, k, v, causal, scale)
        o2, l2 = head_forward(q2, k2, v, causal, scale)
        assert np.abs(o1 - o2).max() < 1e-12
        assert np.abs((l2 - l1) - c).max() < 1e-12


# ------------------------------------------------------------------ P4, P6: closed forms

def test_causal_row_zero_is_v0():
    q, k, v = rand((4, 2, 11, 8), 7), rand((4, 1, 11, 8), 8), rand((4, 1, 11, 8), 9)
    o, lse = attention_forward(q, k, v, True, 0.3)
    for b in range(4):
        for h in range(2):
            assert np.array_equal(o[b, h, 0], v[b, 0, 0])
            assert lse[b, h, 0] == pytest.approx(0.3 * float(q[b, h, 0] @ k[b, 0, 0]), abs=1e-14)


def test_zero_queries_give_uniform_average():
    n, d = 23, 5
    k, v = rand((n, d), 10), rand((n, d), 11)
    q = np.zeros((n, d))
    o, lse = head_forward(q, k, v, True, 1.0)
    for i in range(n):
        assert np.abs(o[i] - v[: i + 1].mean(axis=0)).max() < 1e-14
        assert lse[i] == pytest.approx(math.log(i + 1), abs=1e-14)
    o, lse = head_forward(q, k, v, False, 1.0)
    assert np.abs(o - v.mean(axis=0)).max() < 1e-14
    assert np.abs(lse - math.log(n)).max() < 1e-14


def test_single_token():
    q, k, v = rand((1, 4), 12), rand((1, 4), 13), rand((1, 4), 14)
    for causal in (True, False):
        o, lse = head_forward(q, k, v, causal, 0.25)
        assert np.array_equal(o, v)
        assert lse[0] == pytest.approx(0.25 * float(q[0] @ k[0]), abs=1e-15)
        dq, dk, dv = head_backward(q, k, v, rand((1, 4), 15), causal, 0.25)
        # with one key, P = 1 and the softmax Jacobian is zero
        assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0


def test_rows_subset_matches_full():
    q, k, v = rand((700, 8), 16), rand((700, 8), 17), rand((700, 8), 18)
    rows = np.array([0, 1, 513, 699, 200])
    o, lse = head_forward(q, k, v, True, 0.4)
    os_, ls_ = head_forward(q, k, v, True, 0.4, rows=rows)
    assert np.abs(o[rows] - os_).max() < 1e-14 and np.abs(lse[rows] - ls_).max() < 1e-14


# ------------------------------------------------------------------ P5: online == two-pass

@pytest.mark.parametrize("bc", [1, 5, 7, 32, 128, 200])
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("causal", [True, False])
def test_online_merged_equals_two_pass(bc, seed, causal):
    # tiles' partial states merged in a seeded tree order reach the two-pass result
    n, d = 133, 16
    q, k, v = rand((n, d), 20, 3.0), rand((n, d), 21, 3.0), rand((n, d), 22)
    o1, l1 = head_forward(q, k, v, causal, 0.25)
    o2, l2 = head_forward_merged(q, k, v, causal, 0.25, bc, seed)
    assert np.abs(o1 - o2).max() <= 1e-12 * max(1.0, np.abs(o1).max())
    assert np.abs(l1 - l2).max() <= 1e-12 * max(1.0, np.abs(l1).max())


def test_online_large_logits():
    # logits around |x| ~ 500 (the long-context stress shape) do not overflow either form
    n, d = 96, 16
    q, k, v = rand((n, d), 23, 8.0), rand((n, d), 24, 8.0), rand((n, d), 25)
    o1, l1 = head_forward(q, k, v, True, 0.25)
    o2, l2 = head_forward_merged(q, k, v, True, 0.25, 32, 3)
    assert np.isfinite(o1).all() and np.abs(l1).max() > 50
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-9


def test_merge_is_the_state_of_the_union_by_hand():
    # one row, scores (0, ln 2 | ln 3) with values (1, 2 | 3): A = {0, ln 2} has
    # m = ln 2, l = 1/2 + 1 = 3/2, a = 1/2 + 2 = 5/2; B = {ln 3} has m = ln 3, l = 1,
    # a = 3; the union has m = ln 3, l = (3/2)(2/3) + 1 = 2, a = (5/2)(2/3) + 3 = 14/3
    # (the three-element example's last state), and output 7/3.
    sa = np.array([[0.0, math.log(2.0)]])
    sb = np.array([[math.log(3.0)]])
    A = tile_state(sa, np.array([[1.0], [2.0]]))
    B = tile_state(sb, np.array([[3.0]]))
    assert A[0][0] == pytest.approx(math.log(2.0), abs=1e-15)
    assert A[1][0] == pytest.approx(1.5, rel=1e-15) and A[2][0, 0] == pytest.approx(2.5, rel=1e-15)
    for m, l, a in (merge_states(A, B), merge_states(B, A)):
        assert m[0] == pytest.approx(math.log(3.0), abs=1e-15)
        assert l[0] == pytest.approx(2.0, rel=1e-15)
        assert a[0, 0] == pytest.approx(14 / 3, rel=1e-15)
        assert a[0, 0] / l[0] == pytest.approx(7 / 3, rel=1e-15)


def test_merge_identity_and_hidden_tile():
    # a tile whose keys are all hidden from a row is the merge's identity for that row
    s = np.array([[-np.inf, -np.inf], [0.5, -np.inf]])
    m, l, a = tile_state(s, np.array([[1.0], [2.0]]))
    assert m[0] == -np.inf and l[0] == 0.0 and a[0, 0] == 0.0
    other = (np.array([0.25, 0.25]), np.array([2.0, 2.0]), np.array([[3.0], [3.0]]))
    m2, l2, a2 = merge_states((m, l, a), other)
    assert m2[0] == 0.25 and l2[0] == 2.0 and a2[0, 0] == 3.0


# ------------------------------------------------------------------ P7: grouped-query heads

def test_gqa_equals_mha_with_repeated_kv():
    b, hq, hkv, n, d = 2, 6, 2, 19, 8
    q, k, v, do = rand((b, hq, n, d), 30), rand((b, hkv, n, d), 31), rand((b, hkv, n, d), 32), \
        rand((b, hq, n, d), 33)
    g = hq // hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)   # heads 0,0,0,1,1,1
    for causal in (True, False):
        o, lse = attention_forward(q, k, v, causal, 0.35)
        o2, lse2 = attention_forward(q, kr, vr, causal, 0.35)
        assert np.abs(o - o2).max() == 0 and np.abs(lse - lse2).max() == 0
        dq, dk, dv = attention_backward(q, k, v, do, causal, 0.35)
        dq2, dk2, dv2 = attention_backward(q, kr, vr, do, causal, 0.35)
        assert np.abs(dq - dq2).max() < 1e-13
        assert np.abs(dk - dk2.reshape(b, hkv, g, n, d).sum(axis=2)).max() < 1e-13
        assert np.abs(dv - dv2.reshape(b, hkv, g, n, d).sum(axis=2)).max() < 1e-13
    # query head 1 must use KV head 0 (contiguous groups), not KV head 1
    o, _ = attention_forward(q, k, v, False, 0.35)
    o_h1, _ = head_forward(q[0, 1], k[0, 0], v[0, 0], False, 0.35)
    assert np.abs(o[0, 1] - o_h1).max() == 0


# ------------------------------------------------------------------ P8: finite differences

@pytest.mark.parametrize("causal", [True, False])
def test_gradients_by_central_differences(causal):
    b, hq, hkv, n, d, scale = 1, 2, 1, 5, 3, 0.6
    q, k, v, do = rand((b, hq, n, d), 40), rand((b, hkv, n, d), 41), rand((b, hkv, n, d), 42), \
        rand((b, hq, n, d), 43)

    def loss(q_, k_, v_):
        o, _ = attention_forward(q_, k_, v_, causal, scale)
        return float((o * do).sum())

    dq, dk, dv = attention_backward(q, k, v, do, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{a + "_": b_ for a, b_ in args_p.items()})
                        - loss(**{a + "_": b_ for a, b_ in args_m.items()})) / (2 * h)
        err = np.abs(num - g) / np.maximum(1.0, np.abs(g))
        assert err.max() < 1e-6, (name, err.max())


# ------------------------------------------------------------------ P9: D identity

def test_rowsum_p_dp_equals_do_dot_o():
    n, d = 41, 8
    q, k, v, do = rand((n, d), 50), rand((n, d), 51), rand((n, d), 52), rand((n, d), 53)
    for causal in (True, False):
        p = head_probs(q, k, causal, 0.5)
        o, _ = head_forward(q, k, v, causal, 0.5)
        dp = do @ v.T
        assert np.abs((p * dp).sum(axis=1) - (do * o).sum(axis=1)).max() < 1e-12


# ------------------------------------------------------------------ P10: brute force

def _brute_head(q, k, v, do, causal, scale):
    """Scalar loops with math.fsum; written independently of the oracle."""
    n, d = len(q), len(q[0])
    s = [[scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in range(n)] for i in range(n)]
    vis = [[(j <= i) or not causal for j in range(n)] for i in range(n)]
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


@pytest.mark.parametrize("n", [1, 2, 5, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_scalar_loops(n, causal):
    d = 3
    q, k, v, do = rand((n, d), 60 + n), rand((n, d), 70 + n), rand((n, d), 80 + n), rand((n, d), 90 + n)
    o, lse = head_forward(q, k, v, causal, 0.8)
    dq, dk, dv = head_backward(q, k, v, do, causal, 0.8)
    bo, bl, bdq, bdk, bdv = _brute_head(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, 0.8)
    for a, bb in ((o, bo), (lse, bl), (dq, bdq), (dk, bdk), (dv, bdv)):
        assert np.abs(a - np.array(bb)).max() <= 1e-13


# ------------------------------------------------------------------ P11: independent library

@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_cpu_float64_sdpa_and_autograd(causal):
    b, hq, hkv, n, d, scale = 2, 4, 2, 33, 16, 0.25
    q, k, v, do = rand((b, hq, n, d), 100), rand((b, hkv, n, d), 101), rand((b, hkv, n, d), 102), \
        rand((b, hq, n, d), 103)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    g = hq // hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1),
        is_causal=causal, scale=scale)
    out.backward(torch.tensor(do))
    o, _ = attention_forward(q, k, v, causal, scale)
    dq, dk, dv = attention_backward(q, k, v, do, causal, scale)
    assert np.abs(o - out.detach().numpy()).max() < 1e-12
    assert np.abs(dq - tq.grad.numpy()).max() < 1e-12
    assert np.abs(dk - tk.grad.numpy()).max() < 1e-12
    assert np.abs(dv - tv.grad.numpy()).max() < 1e-12


# ------------------------------------------------------------------ process pool and heads subset

def test_pool_and_subsets_match_serial():
    b, hq, hkv, n, d = 2, 4, 2, 40, 8
    q, k, v, do = rand((b, hq, n, d), 110), rand((b, hkv, n, d), 111), rand((b, hkv, n, d), 112), \
        rand((b, hq, n, d), 113)
    o, lse = attention_forward(q, k, v, True, 0.3)
    o2, lse2 = attention_forward(q, k, v, True, 0.3, workers=2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    o3, _ = attention_forward(q, k, v, True, 0.3, heads=[(1, 3)])
    assert np.array_equal(o3[1, 3], o[1, 3]) and np.isnan(o3[0, 0]).all()
    dq, dk, dv = attention_backward(q, k, v, do, True, 0.3)
    dq2, dk2, dv2 = attention_backward(q, k, v, do, True, 0.3, groups=[(1, 1)], workers=2)
    assert np.abs(dq2[1, 2:] - dq[1, 2:]).max() == 0 and np.isnan(dq2[1, :2]).all()
    assert np.abs(dk2[1, 1] - dk[1, 1]).max() < 1e-15 and np.abs(dv2[1, 1] - dv[1, 1]).max() < 1e-15
