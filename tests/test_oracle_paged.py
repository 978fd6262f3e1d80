"""Pins of the oracle's paged key/value cache: logical token t of sequence b lives in
page block_table[b, t // P] at row t % P (P tokens per page).

Pinned by an identity table over a contiguous cache (the pinned decode oracle),
scalar loops that walk the table token by token, independence from where the pages
sit in the pool, per-sequence lengths against each sequence's own prefix, and a
planted mistake in the page arithmetic.
"""
import numpy as np
import pytest

import oracle.attention as A
from oracle import decode_forward, paged_decode_forward, paged_gather


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def to_pages(kv, psize, perm):
    """Contiguous [B, Hkv, Nk, d] -> pool [B * Nk/P, Hkv, P, d] placed by perm, and the table."""
    B, H, N, d = kv.shape
    nb = N // psize
    pool = np.zeros((B * nb, H, psize, d))
    table = np.zeros((B, nb), dtype=np.int64)
    for b in range(B):
        for i in range(nb):
            p = perm[b * nb + i]
            pool[p] = kv[b, :, i * psize:(i + 1) * psize, :]
            table[b, i] = p
    return pool, table


@pytest.mark.parametrize("causal", [True, False])
def test_identity_table_is_the_contiguous_decode(causal):
    B, Hq, Hkv, Nq, N, d, P = 2, 4, 2, 3, 24, 5, 8
    q, k, v = rand((B, Hq, Nq, d), 1), rand((B, Hkv, N, d), 2), rand((B, Hkv, N, d), 3)
    kp, table = to_pages(k, P, np.arange(B * N // P))
    vp, _ = to_pages(v, P, np.arange(B * N // P))
    o, lse = paged_decode_forward(q, kp, vp, table, [N] * B, causal, 0.6)
    o2, lse2 = decode_forward(q, k, v, causal, 0.6)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_pool_placement_does_not_matter():
    B, Hq, Hkv, Nq, N, d, P = 3, 2, 1, 2, 32, 4, 8
    q, k, v = rand((B, Hq, Nq, d), 4), rand((B, Hkv, N, d), 5), rand((B, Hkv, N, d), 6)
    ident = [to_pages(x, P, np.arange(B * N // P)) for x in (k, v)]
    perm = np.random.default_rng(7).permutation(B * N // P)
    shuf = [to_pages(x, P, perm) for x in (k, v)]
    o1, l1 = paged_decode_forward(q, ident[0][0], ident[1][0], ident[0][1], [N] * B, True, 0.5)
    o2, l2 = paged_decode_forward(q, shuf[0][0], shuf[1][0], shuf[0][1], [N] * B, True, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert not np.array_equal(ident[0][0], shuf[0][0])


def test_gather_walks_the_table_token_by_token():
    # scalar loops: token t of sequence b is row t % P of page table[b][t // P]
    Hkv, P, d, npages = 2, 4, 3, 7
    pool = rand((npages, Hkv, P, d), 8)
    table = np.array([[5, 0, 3], [6, 2, 1]])
    for b, n in ((0, 11), (1, 9)):
        g = paged_gather(pool, table, n, b)
        for h in range(Hkv):
            for t in range(n):
                page = int(table[b][t // P])
                for c in range(d):
                    assert g[h, t, c] == pool[page, h, t % P, c]


@pytest.mark.parametrize("causal", [True, False])
def test_each_sequence_sees_only_its_own_length(causal):
    B, Hq, Hkv, Nq, d, P, nb = 3, 2, 1, 2, 4, 8, 4
    lens = [5, 32, 17]
    q = rand((B, Hq, Nq, d), 9)
    k, v = rand((B, Hkv, nb * P, d), 10), rand((B, Hkv, nb * P, d), 11)
    perm = np.random.default_rng(12).permutation(B * nb)
    kp, table = to_pages(k, P, perm)
    vp, _ = to_pages(v, P, perm)
    o, lse = paged_decode_forward(q, kp, vp, table, lens, causal, 0.7)
    for b, n in enumerate(lens):
        ob, lb = decode_forward(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], causal, 0.7)
        assert np.array_equal(o[b:b + 1], ob) and np.array_equal(lse[b:b + 1], lb)


def test_planted_page_arithmetic_mistake_is_caught(monkeypatch):
    # row t // P of page t % P (the two indices swapped) must break the identity pin
    def wrong(pages, block_table, seq_len, b):
        pages = np.asarray(pages, dtype=np.float64)
        table = np.asarray(block_table)
        psize = pages.shape[2]
        tok = np.arange(seq_len)
        return np.transpose(pages[table[b, tok % psize], :, tok // psize, :], (1, 0, 2))
    monkeypatch.setattr(A, "paged_gather", wrong)
    # (several causal queries over a partial length, so that the keys a row sees change;
    # a single query over the whole cache would not notice a permutation of tokens)
    B, Hq, Hkv, Nq, N, d, P, n = 1, 2, 1, 3, 16, 3, 4, 14
    q, k, v = rand((B, Hq, Nq, d), 13), rand((B, Hkv, N, d), 14), rand((B, Hkv, N, d), 15)
    kp, table = to_pages(k, P, np.arange(N // P))
    vp, _ = to_pages(v, P, np.arange(N // P))
    o, _ = A.paged_decode_forward(q, kp, vp, table, [n], True, 0.6)
    o2, _ = decode_forward(q, k[:, :, :n], v[:, :, :n], True, 0.6)
    assert np.abs(o - o2).max() > 1e-6
