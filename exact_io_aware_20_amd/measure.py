"""Algorithmic FLOP and byte model used by the benchmark's roofline figures.

* Compute stays Theta(N^2 d) under the method (page "ZeRO 与 FlashAttention 各优化什么?",
  section "FlashAttention 与 ZeRO 必须分开": the dense FLOPs do not become linear).
  Forward = two N x N x d contractions (S = Q K^T and O = P V) = 4 B Hq N^2 d flop,
  halved for causal attention.
* Backward = 2.5 x forward: five N x N x d contractions (recomputed S, dP, dV, dK,
  dQ) against the forward's two, in the 2.2-2.5x range that the interview bank
  ch.029 question #36 gives for FlashAttention's backward.
* Compulsory HBM traffic: every input read once and every output written once;
  nothing of size N x N (the score matrix never reaches HBM).
* The score-matrix sizes the pages quote (code-corey Q38 section 1: 8K x 8K x 4 B
  ~ 256 MB; interview bank #36 section 2: 32 x 4096 x 4096 x 4 B ~ 2.1 GB) and the
  KV saving of grouped-query attention (lecture summary section "减少缓存表示并验证草稿":
  24 query heads over 2 KV groups, about 91 %) are reproduced by the helpers below.
"""
from __future__ import annotations

# MI355X published peaks (AMD specifications): dense bf16 MFMA, fp32 vector and HBM3E.
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def fwd_flops(B, Hq, N, d, causal: bool) -> float:
    f = 4.0 * B * Hq * N * N * d
    return f / 2 if causal else f


def bwd_flops(B, Hq, N, d, causal: bool) -> float:
    return 2.5 * fwd_flops(B, Hq, N, d, causal)


def fwd_bytes(B, Hq, Hkv, N, d, elt: int) -> int:
    """Read Q, K, V once; write O and the fp32 LSE once."""
    return elt * (2 * B * Hq * N * d + 2 * B * Hkv * N * d) + 4 * B * Hq * N


def bwd_bytes(B, Hq, Hkv, N, d, elt: int) -> int:
    """Read Q, O, dO, K, V, LSE; write dQ, dK, dV; the two fp32 per-row terms (D and
    LSE in base 2) written once and read by the dK/dV and dQ kernels."""
    q_sized = B * Hq * N * d
    kv_sized = B * Hkv * N * d
    return elt * (3 * q_sized + 2 * kv_sized) + 4 * B * Hq * N \
        + elt * (q_sized + 2 * kv_sized) + 3 * 2 * 4 * B * Hq * N


def preprocess_bytes(B, Hq, N, d, elt: int, zero_acc: bool = False) -> int:
    """The backward preprocess reads O, dO and the fp32 LSE and writes two fp32 per row
    (D and LSE in base 2), and for the fused backward zeroes the fp32 dQ accumulator
    (d values per row)."""
    return 2 * elt * B * Hq * N * d + 3 * 4 * B * Hq * N + (4 * B * Hq * N * d if zero_acc else 0)


def dq_convert_bytes(B, Hq, N, d, elt: int) -> int:
    """The conversion of the fused backward's fp32 dQ accumulator to the output dtype:
    reads d fp32 values per query row, writes d elements."""
    return (4 + elt) * B * Hq * N * d


def score_matrix_bytes(N, elt: int = 4, heads: int = 1, batch: int = 1) -> int:
    """Size of one materialised N x N score matrix per head (what the method avoids)."""
    return batch * heads * N * N * elt


def kv_storage_saving(Hq, Hkv) -> float:
    """Fraction of K/V storage saved by Hkv shared heads versus Hq (MHA)."""
    return 1.0 - Hkv / Hq


def decode_bytes(B, Hq, Hkv, Nq, Nk, d, elt: int) -> int:
    """Decode call: read Q and the K/V cache once, write O and the fp32 LSE once."""
    return elt * (2 * B * Hq * Nq * d + 2 * B * Hkv * Nk * d) + 4 * B * Hq * Nq


def decode_split_bytes(B, Hq, Hkv, Nq, Nk, d, elt: int) -> int:
    """The split kernel's algorithmic traffic: Q and the K/V cache read once (per
    (batch, KV head, key) unit: 2 d elt bytes of K and V)."""
    return elt * (B * Hq * Nq * d + 2 * B * Hkv * Nk * d)


def decode_flops(B, Hq, Nq, Nk, d) -> float:
    """Two Nq x Nk x d contractions per query head (the causal mask hides at most
    Nq - 1 keys of Nk, so the full count is used)."""
    return 4.0 * B * Hq * Nq * Nk * d


def visible_pairs(N, causal: bool, window: int = -1) -> int:
    """Number of (query, key) pairs with key j visible to query i: j <= i when causal,
    |i - j| <= window when window >= 0 (exact count, no halving convention)."""
    w = N if window < 0 else window
    total = 0
    for i in range(N):
        lo = max(0, i - w)
        hi = i if causal else min(N - 1, i + w)
        total += hi - lo + 1
    return total


def window_fwd_flops(B, Hq, N, d, causal: bool, window: int) -> float:
    """Forward of a sliding-window call: two contractions over the visible pairs."""
    return 4.0 * B * Hq * d * visible_pairs(N, causal, window)


def paged_decode_bytes(seq_lens, B, Hq, Hkv, Nq, d, elt: int, max_blocks: int) -> int:
    """Paged decode call: every cached token of every sequence (K and V of each KV
    head) read once, Q read and O, LSE written once, the block table and lengths read."""
    tokens = int(sum(int(n) for n in seq_lens))
    return elt * (2 * B * Hq * Nq * d + 2 * Hkv * tokens * d) + 4 * B * Hq * Nq + 4 * B * (max_blocks + 1)


def paged_split_bytes(seq_lens, B, Hq, Hkv, Nq, d, elt: int) -> int:
    """The paged split kernel's algorithmic traffic: Q and the cached K/V read once."""
    tokens = int(sum(int(n) for n in seq_lens))
    return elt * (B * Hq * Nq * d + 2 * Hkv * tokens * d)


def layout_pairs(N, layout, causal: bool, block: int = 64) -> int:
    """Visible (query, key) pairs under a block-sparse layout [nb][nb] (and the causal
    rule): each set block pair contributes its rows x keys, or rows(rows+1)/2 on the
    diagonal under the causal rule and nothing above it."""
    import numpy as np
    lay = np.asarray(layout).astype(bool)
    nb = lay.shape[0]
    size = np.minimum(block, N - block * np.arange(nb))
    total = 0
    for i in range(nb):
        for j in np.nonzero(lay[i])[0]:
            if causal and j > i:
                continue
            if causal and j == i:
                total += int(size[i]) * (int(size[i]) + 1) // 2
            else:
                total += int(size[i]) * int(size[j])
    return total


def layout_fwd_flops(B, Hq, N, d, causal: bool, layout) -> float:
    """Forward of a block-sparse call: two contractions over the visible pairs."""
    return 4.0 * B * Hq * d * layout_pairs(N, layout, causal)
