"""CPU float64 oracle for exact scaled dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY. The tests, the package's ``smoke()`` check and the
CPU-baseline leg of the benchmark may import this module; the HIP library and its
Python binding never do. It shares no code, tables or helpers with the GPU path.

What it computes is the plain definition of attention, written out:

    S = scale * Q K^T            (one query head against the KV head of its group)
    S_ij = -inf  where j > i     (causal: a token sees itself and earlier tokens)
    P = softmax(S) row-wise,  O = P V,  LSE_i = log sum_j exp(S_ij)

Sources, cited by page title and section:

* "ZeRO 与 FlashAttention 各优化什么?" (wushixiongai.com), section
  "注意力瓶颈与优化路线": FlashAttention / fused SDPA computes *exact* dense attention;
  tiling, online softmax and fusion change only where and in which order it is computed.
* Stanford lecture summary (youtublog.net), section "GPU 显存和注意力瓶颈": in causal
  self-attention each token attends to itself and the tokens before it (mask j <= i,
  diagonal included).  Section "推导 FlashAttention 的在线 softmax": an output row is a
  numerator (sum of exp(score) * value) over a denominator (sum of exp(score)); the
  method keeps a small per-row statistic for the backward pass.  Section
  "减少缓存表示并验证草稿": H query heads share G key/value heads (G = H is MHA, G = 1
  is MQA).
* "LLM interview question bank" ch.029 (ricardokevins.github.io), question #36
  "FlashAttention 为什么常被说成是 IO-aware", section 2: Q, K, V live in R^(B x H x L x d).

Readings where the pages are silent (each listed with its reason in the design notes):

* The scale is the caller's (configs pass 1/sqrt(d)).
* The saved statistic is the natural-log log-sum-exp of the *scaled* logits.
* Query head hq uses KV head hq // (Hq / Hkv) (contiguous groups).
* Decoding against a key/value cache (``decode_forward``): the Nq queries are the
  last Nq tokens of a sequence whose Nk keys and values, their own included, are all
  in the cache (lecture summary, section "衡量并优化推理": decoding reuses the keys
  and values of earlier tokens instead of recomputing them).  Query i therefore sits
  at position Nk - Nq + i, and causally sees keys j <= Nk - Nq + i; with Nq = Nk
  this is the ordinary causal mask.
* Sliding window (``window`` >= 0; page "ZeRO 与 FlashAttention 各优化什么?", section
  "注意力瓶颈与优化路线": a sliding window restricts which positions a query sees):
  query position i sees key j only if |i - j| <= window, on top of the causal rule,
  so a causal row sees its window + 1 most recent keys.  window < 0 means no window.
* Block-sparse layout (``block_mask``, same page and section: block-sparse and
  global + local patterns compute only part of the positions): a 0/1 matrix over
  BLOCK x BLOCK blocks of (query, key) positions, shared by every head; query i sees
  key j only if block_mask[i // BLOCK][j // BLOCK] is set, on top of the causal rule.
  A row that sees no key gets O = 0 and LSE = -inf.
* The gradients are the analytic softmax-Jacobian gradients (the pages print none):
      dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
      dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
  with dK and dV of a KV head summed over the query heads of its group.

Rows are processed in blocks, but each block holds *full* rows of S and P
(the two-pass softmax of the definition, not an online one), so nothing here is
blocked, fused or reordered beyond what a BLAS matmul does internally.
"""
from __future__ import annotations

import contextlib
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROW_BLOCK = 512
BLOCK = 64   # side of a block of the block-sparse layout


def _f64(x) -> np.ndarray:
    """Upcast anything array-like (numpy or a CPU torch tensor) to float64 numpy."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype, go via float32
        x = x.detach().to("cpu")
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _scores(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray, causal: bool, scale: float, window: int = -1,
            block_mask=None):
    """S for the given query rows against all keys, with the causal mask (key <= query)
    and, for window >= 0, the sliding-window mask (|query - key| <= window) applied.

    ``rows`` are the queries' positions in the key sequence."""
    s = scale * (q_rows @ k.T)
    cols = np.arange(k.shape[0])
    if causal:
        s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
    if window >= 0:
        s = np.where(np.abs(cols[None, :] - rows[:, None]) <= window, s, -np.inf)
    if block_mask is not None:
        bm = np.asarray(block_mask, dtype=bool)
        s = np.where(bm[rows[:, None] // BLOCK, cols[None, :] // BLOCK], s, -np.inf)
    return s


def _query_offset(nq: int, nk: int) -> int:
    """Position of query row 0 in the key sequence: the queries are its last nq tokens."""
    return nk - nq


def head_forward(q, k, v, causal: bool, scale: float, rows=None, offset: int = 0, window: int = -1,
                 block_mask=None):
    """One query head: O and LSE for the selected query rows (default: all rows).

    q: [Nq, d]; k, v: [Nk, d] (the KV head of this query's group); query row i sits
    at position i + offset of the key sequence (offset 0 when queries and keys are
    the same sequence); ``window`` >= 0 adds the sliding-window mask.  Returns
    (O [len(rows), d], LSE [len(rows)]) in float64.  A
    row with no visible key (not reachable when the queries are the tail of the key
    sequence) gives O = 0 and LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.full(rows.size, -np.inf)
    for b0 in range(0, rows.size, ROW_BLOCK):
        r = rows[b0:b0 + ROW_BLOCK]
        s = _scores(q[r], k, r + offset, causal, scale, window, block_mask)
        m = s.max(axis=1)                              # pass 1: row max
        ok = np.isfinite(m)
        e = np.exp(s - np.where(ok, m, 0.0)[:, None])  # pass 2: exponentials
        l = e.sum(axis=1)
        p = e / np.where(ok, l, 1.0)[:, None]
        o[b0:b0 + r.size] = np.where(ok[:, None], p @ v, 0.0)
        lse[b0:b0 + r.size] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), -np.inf)
    return o, lse


def head_probs(q, k, causal: bool, scale: float, window: int = -1, block_mask=None):
    """The full softmax matrix P [N, N] of one head (small inputs only)."""
    q, k = _f64(q), _f64(k)
    rows = np.arange(q.shape[0])
    s = _scores(q, k, rows, causal, scale, window, block_mask)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def head_backward(q, k, v, do, causal: bool, scale: float, window: int = -1, block_mask=None):
    """One query head: (dQ, dK, dV) for L = sum(dO * O), float64.

    dK and dV are this head's contribution to its KV head; the caller sums them
    over the query heads of a group.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b0 in range(0, n, ROW_BLOCK):
        r = np.arange(b0, min(n, b0 + ROW_BLOCK))
        s = _scores(q[r], k, r, causal, scale, window, block_mask)
        m = s.max(axis=1, keepdims=True)
        ok = np.isfinite(m)                           # rows that see no key have P = 0
        e = np.exp(s - np.where(ok, m, 0.0))
        p = e / np.where(ok, e.sum(axis=1, keepdims=True), 1.0)   # P, full rows
        dp = do[r] @ v.T                              # dP = dO V^T
        dvec = (p * dp).sum(axis=1, keepdims=True)    # D_i = sum_j P_ij dP_ij
        ds = p * (dp - dvec)                          # dS = P * (dP - D)
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
        dv += p.T @ do[r]
    return dq, dk, dv


# --------------------------------------------------------------------------- batched

def _group(hq: int, hq_total: int, hkv_total: int) -> int:
    """KV head used by query head hq: contiguous groups of Hq/Hkv query heads."""
    return hq // (hq_total // hkv_total)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays")
    b, hq, n, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[2] != n or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if hq % k.shape[1] != 0:
        raise ValueError("Hq must be a multiple of Hkv")


def _fwd_unit(args):
    q, k, v, causal, scale, rows, offset, window, block_mask = args
    return head_forward(q, k, v, causal, scale, rows, offset, window, block_mask)


def _bwd_unit(args):
    q, k, v, do, causal, scale, window, block_mask = args
    return head_backward(q, k, v, do, causal, scale, window, block_mask)


@contextlib.contextmanager
def _pool(workers: int):
    """Process pool of fresh interpreters (spawn), one BLAS thread each."""
    keys = ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    os.environ.update({k: "1" for k in keys})
    try:
        with ProcessPoolExecutor(max_workers=workers,
                                 mp_context=multiprocessing.get_context("spawn")) as ex:
            yield ex
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _run(fn, jobs, workers: int):
    if workers > 1 and len(jobs) > 1:
        with _pool(min(workers, len(jobs))) as ex:
            return list(ex.map(fn, jobs))
    return [fn(j) for j in jobs]


def attention_forward(q, k, v, causal: bool, scale: float, heads=None, rows=None, workers: int = 1,
                      window: int = -1, block_mask=None):
    """O [B,Hq,N,d] and LSE [B,Hq,N] (float64) for every (b, hq) in ``heads``.

    ``heads`` is an iterable of (b, hq) pairs (default: all); entries of heads not
    listed are NaN.  ``rows`` optionally restricts the computed query rows (the same
    rows for every listed head).  ``workers`` > 1 runs heads in a process pool.
    ``window`` >= 0 adds the sliding-window mask |i - j| <= window; ``block_mask`` (a
    0/1 matrix over BLOCK x BLOCK blocks) the block-sparse layout.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check_shapes(q, k, v)
    b_, hq_, n, d = q.shape
    hkv_ = k.shape[1]
    heads = [(b, h) for b in range(b_) for h in range(hq_)] if heads is None else list(heads)
    o = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    bm = None if block_mask is None else np.asarray(block_mask, dtype=bool)
    jobs = [(q[b, h], k[b, _group(h, hq_, hkv_)], v[b, _group(h, hq_, hkv_)], causal, scale, rows, 0, window, bm)
            for b, h in heads]
    results = _run(_fwd_unit, jobs, workers)
    sel = slice(None) if rows is None else np.asarray(rows)
    for (b, h), (ob, lb) in zip(heads, results):
        o[b, h, sel] = ob
        lse[b, h, sel] = lb
    return o, lse


def attention_backward(q, k, v, do, causal: bool, scale: float, groups=None, workers: int = 1,
                       window: int = -1, block_mask=None):
    """dQ [B,Hq,N,d], dK and dV [B,Hkv,N,d] (float64) for the listed (b, hkv) groups.

    A group's dK/dV is the sum over its Hq/Hkv query heads; the dQ of every query
    head in a listed group is filled.  Entries outside the listed groups are NaN.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _check_shapes(q, k, v)
    b_, hq_, n, d = q.shape
    hkv_ = k.shape[1]
    g = hq_ // hkv_
    groups = [(b, h) for b in range(b_) for h in range(hkv_)] if groups is None else list(groups)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    units = [(b, hk, h) for b, hk in groups for h in range(hk * g, hk * g + g)]
    bm = None if block_mask is None else np.asarray(block_mask, dtype=bool)
    jobs = [(q[b, h], k[b, hk], v[b, hk], do[b, h], causal, scale, window, bm) for b, hk, h in units]
    results = _run(_bwd_unit, jobs, workers)
    for b, hk in groups:
        dk[b, hk] = 0.0
        dv[b, hk] = 0.0
    for (b, hk, h), (dqh, dkh, dvh) in zip(units, results):
        dq[b, h] = dqh
        dk[b, hk] += dkh
        dv[b, hk] += dvh
    return dq, dk, dv


def decode_forward(q, k, v, causal: bool, scale: float, heads=None, workers: int = 1):
    """Attention of Nq new queries against a key/value cache of Nk tokens.

    q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d].  The queries are the last Nq tokens of the
    sequence, so query i sits at position Nk - Nq + i and, when causal, sees the
    keys j <= Nk - Nq + i.  Returns O [B,Hq,Nq,d] and LSE [B,Hq,Nq] (float64) for
    every (b, hq) in ``heads`` (default: all; other entries NaN).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays")
    b_, hq_, nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b_ or k.shape[3] != d or hq_ % k.shape[1] != 0:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    hkv_, nk = k.shape[1], k.shape[2]
    heads = [(b, h) for b in range(b_) for h in range(hq_)] if heads is None else list(heads)
    off = _query_offset(nq, nk)
    o = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    jobs = [(q[b, h], k[b, _group(h, hq_, hkv_)], v[b, _group(h, hq_, hkv_)], causal, scale, None, off, -1, None)
            for b, h in heads]
    for (b, h), (ob, lb) in zip(heads, _run(_fwd_unit, jobs, workers)):
        o[b, h] = ob
        lse[b, h] = lb
    return o, lse


def paged_gather(pages, block_table, seq_len: int, b: int):
    """The first ``seq_len`` tokens of sequence b from a paged pool, contiguous.

    pages [num_pages, Hkv, P, d]: page p holds P consecutive tokens of every KV head;
    block_table[b, i] is the page holding the sequence's tokens i*P .. i*P + P - 1
    (lecture summary, "衡量并优化推理": metadata maps logical token positions to
    physical blocks).  Returns [Hkv, seq_len, d].
    """
    pages = _f64(pages)
    table = np.asarray(block_table, dtype=np.int64)
    psize = pages.shape[2]
    tok = np.arange(seq_len)
    phys = table[b, tok // psize]
    return np.transpose(pages[phys, :, tok % psize, :], (1, 0, 2))


def paged_decode_forward(q, k_pages, v_pages, block_table, seq_lens, causal: bool, scale: float,
                         workers: int = 1):
    """Decode against a paged key/value cache: sequence b's Nk_b = seq_lens[b] cached
    tokens are gathered through the block table, then attended exactly as
    ``decode_forward`` (its Nq queries at positions Nk_b - Nq + i).  q [B,Hq,Nq,d].
    Returns O [B,Hq,Nq,d] and LSE [B,Hq,Nq] (float64)."""
    q = _f64(q)
    o = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    for b in range(q.shape[0]):
        n = int(seq_lens[b])
        kb = paged_gather(k_pages, block_table, n, b)[None]
        vb = paged_gather(v_pages, block_table, n, b)[None]
        o[b:b + 1], lse[b:b + 1] = decode_forward(q[b:b + 1], kb, vb, causal, scale, workers=workers)
    return o, lse
