"""The FLOP/byte model reproduces the sizes the pages quote (closed forms)."""
import pytest

from exact_io_aware_20_amd import measure


def test_score_matrix_8k_fp32_is_256_mib():
    # code-corey Q38, section 1: 8K x 8K x 4 B ~ 256 MB for one score matrix
    assert measure.score_matrix_bytes(8192, 4) == 268_435_456 == 256 * 2**20


def test_scores_b1_h32_l4096_is_2_1_gb():
    # interview bank ch.029 #36, section 2: 32 x 4096 x 4096 x 4 B ~ 2.1 GB
    assert measure.score_matrix_bytes(4096, 4, heads=32, batch=1) == 2_147_483_648


def test_gqa_24_over_2_saves_about_91_percent():
    # lecture summary, section on grouped-query attention: 24 query heads, 2 KV groups
    assert measure.kv_storage_saving(24, 2) == pytest.approx(0.9167, abs=1e-4)


def test_flop_convention():
    f = measure.fwd_flops(2, 32, 8192, 128, causal=True)
    assert f == pytest.approx(1.0995e12, rel=1e-4)
    assert measure.fwd_flops(1, 1, 256, 64, causal=False) == 4 * 256 * 256 * 64
    assert measure.bwd_flops(2, 32, 8192, 128, True) == 2.5 * f


def test_compulsory_bytes():
    # read q,k,v and write o (bf16) plus fp32 lse
    assert measure.fwd_bytes(1, 1, 1, 256, 64, 4) == 4 * 4 * 256 * 64 + 4 * 256
    b = measure.fwd_bytes(8, 24, 2, 4096, 128, 2)
    assert b == 2 * (2 * 8 * 24 * 4096 * 128 + 2 * 8 * 2 * 4096 * 128) + 4 * 8 * 24 * 4096


def test_visible_pairs_closed_forms():
    from exact_io_aware_20_amd import measure
    for n in (1, 5, 64, 300):
        assert measure.visible_pairs(n, True) == n * (n + 1) // 2
        assert measure.visible_pairs(n, False) == n * n
        assert measure.visible_pairs(n, True, 0) == n and measure.visible_pairs(n, False, 0) == n
        for w in (1, 7, 63):
            if n > w:   # causal: rows i >= w see w + 1 keys, rows i < w see i + 1
                assert measure.visible_pairs(n, True, w) == n * (w + 1) - w * (w + 1) // 2
                assert measure.visible_pairs(n, False, w) == 2 * measure.visible_pairs(n, True, w) - n


def test_layout_pairs_closed_forms():
    import numpy as np
    from exact_io_aware_20_amd import measure
    for n in (64, 130, 300):
        nb = -(-n // 64)
        ones = np.ones((nb, nb), bool)
        assert measure.layout_pairs(n, ones, False) == n * n
        assert measure.layout_pairs(n, ones, True) == n * (n + 1) // 2
        assert measure.layout_pairs(n, np.eye(nb, dtype=bool), False) == sum(min(64, n - 64 * i) ** 2 for i in range(nb))
        assert measure.layout_pairs(n, np.zeros((nb, nb), bool), True) == 0
