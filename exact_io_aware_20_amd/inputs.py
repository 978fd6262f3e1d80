"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws iid N(0, 1) tensors from
seeded CPU generators and casts them to the run dtype (round to nearest even), so
that the HIP path and the CPU oracle see bit-identical values.

Workloads (the seed base of workload w is 1000*w; q, k, v, dO add 1, 2, 3, 4):

==========================  ====  ===  ===  =====  ===  ======  =====  ===========
name                         B    Hq   Hkv    N     d   causal  dtype  passes
==========================  ====  ===  ===  =====  ===  ======  =====  ===========
tiny_f32                      1     1    1    256   64  no      f32    fwd
causal_n2048_d64              4    16   16   2048   64  yes     bf16   fwd (+LSE)
causal_n8192_d128             2    32   32   8192  128  yes     bf16   fwd, bwd
gqa_n4096_d128                8    24    2   4096  128  yes     bf16   fwd, bwd
longctx_n65536_d128           1    16   16  65536  128  both    bf16   fwd
decode_gqa_kv65536_d128       8    24    2  65536  128  yes     bf16   decode, Nq=1
decode_spec4_kv65536_d128     8    24    2  65536  128  yes     bf16   decode, Nq=4
window_n16384_w2047_d128      2    16   16  16384  128  yes     bf16   fwd, bwd (window 2047)
decode_paged_kv65536_d128    16    24    2  65536  128  yes     bf16   paged decode, Nq=1
blocksparse_n16384_d128       2    16   16  16384  128  yes     bf16   fwd, bwd (local + global)
==========================  ====  ===  ===  =====  ===  ======  =====  ===========

The long-context workload multiplies q and k by 8 before the cast (a power of two,
exact in bf16), so logits reach |x| ~ 500 and stress the running-max rescaling.
The decode workloads hold a cache of N = 65536 keys and values per KV head and
Nq = 1 (one new token) or Nq = 4 (four tokens checked at once) queries per query
head; q is [B, Hq, Nq, d] and k, v are [B, Hkv, N, d].  The window workload lets each
query see only keys within 2047 positions (with the causal rule: its 2048 most recent
tokens, itself included).  The paged decode workload holds 16 sequences of seeded
lengths between 2048 and 65536 tokens (the first exactly 65536) in 256-token pages
scattered over a pool by a seeded permutation; unused table entries are -1.  The
block-sparse workload's layout over 64 x 64 blocks is local + global: a query block
sees its own block and the 7 before it, and the first 2 key blocks.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed_base: int
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: tuple          # causal settings run on this shape
    dtype: str             # "bf16" or "f32"
    backward: bool
    qk_mult: float = 1.0
    extra: dict = field(default_factory=dict)
    nq: int = 0            # decode: query rows per head (0: the queries are the whole sequence)
    window: int = -1       # sliding window |i - j| <= window (-1: none)
    page_size: int = 0     # paged decode: tokens per page (0: contiguous cache); N is the longest sequence
    layout: tuple = ()     # block-sparse: (local blocks, global blocks) of local_global_layout

    @property
    def decode(self) -> bool:
        return self.nq > 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny_f32", 1000, 1, 1, 1, 256, 64, (False,), "f32", False),
        Workload("causal_n2048_d64", 2000, 4, 16, 16, 2048, 64, (True,), "bf16", False),
        Workload("causal_n8192_d128", 3000, 2, 32, 32, 8192, 128, (True,), "bf16", True),
        Workload("gqa_n4096_d128", 4000, 8, 24, 2, 4096, 128, (True,), "bf16", True),
        Workload("longctx_n65536_d128", 5000, 1, 16, 16, 65536, 128, (True, False), "bf16",
                 False, qk_mult=8.0),
        Workload("decode_gqa_kv65536_d128", 6000, 8, 24, 2, 65536, 128, (True,), "bf16", False, nq=1),
        Workload("decode_spec4_kv65536_d128", 7000, 8, 24, 2, 65536, 128, (True,), "bf16", False, nq=4),
        Workload("window_n16384_w2047_d128", 8000, 2, 16, 16, 16384, 128, (True,), "bf16", True, window=2047),
        Workload("decode_paged_kv65536_d128", 9000, 16, 24, 2, 65536, 128, (True,), "bf16", False, nq=1,
                 page_size=256),
        Workload("blocksparse_n16384_d128", 10000, 2, 16, 16, 16384, 128, (True,), "bf16", True, layout=(8, 2)),
    )
}


def seeded_normal(shape, seed: int, dtype=torch.bfloat16, mult: float = 1.0) -> torch.Tensor:
    """iid N(0,1) drawn in float32 from ``torch.Generator().manual_seed(seed)``,
    multiplied by ``mult`` and cast to ``dtype``.  Always a CPU tensor."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(dtype)


def make_inputs(B, Hq, Hkv, N, d, seed_base: int, dtype=torch.bfloat16, qk_mult: float = 1.0,
                with_do: bool = False, nq: int = 0) -> dict:
    """q [B,Hq,Nq,d], k and v [B,Hkv,N,d] (and dO like q) on the CPU; Nq = nq, or N
    when nq is 0."""
    nq = nq or N
    out = {
        "q": seeded_normal((B, Hq, nq, d), seed_base + 1, dtype, qk_mult),
        "k": seeded_normal((B, Hkv, N, d), seed_base + 2, dtype, qk_mult),
        "v": seeded_normal((B, Hkv, N, d), seed_base + 3, dtype),
    }
    if with_do:
        out["do"] = seeded_normal((B, Hq, nq, d), seed_base + 4, dtype)
    return out


def workload_inputs(w: Workload, with_do: bool | None = None) -> dict:
    return make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed_base, w.torch_dtype, w.qk_mult,
                       w.backward if with_do is None else with_do, w.nq)


def paged_cache(B, Hq, Hkv, Nq, max_len, d, page_size, seed_base: int, min_len: int = 1, lens=None,
                spare_pages: int = 0, dtype=torch.bfloat16) -> dict:
    """A paged decode call on the CPU: q [B,Hq,Nq,d]; pools k_pages, v_pages
    [num_pages,Hkv,page_size,d]; block_table int32 [B, ceil(max_len/page_size)] with -1
    in unused entries; seq_lens int32 [B].  Lengths are drawn from [min_len, max_len]
    (the first is max_len) unless given; each sequence's pages are placed in the pool
    by a seeded permutation."""
    import numpy as np
    rng = np.random.default_rng(seed_base + 5)
    if lens is None:
        lens = rng.integers(min_len, max_len + 1, size=B)
        lens[0] = max_len
    lens = np.asarray(lens, dtype=np.int64)
    max_blocks = (max_len + page_size - 1) // page_size
    need = (lens + page_size - 1) // page_size
    num_pages = max(1, int(need.sum()) + spare_pages)
    perm = rng.permutation(num_pages)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        table[b, :need[b]] = perm[nxt:nxt + need[b]]
        nxt += int(need[b])
    return {
        "q": seeded_normal((B, Hq, Nq, d), seed_base + 1, dtype),
        "k_pages": seeded_normal((num_pages, Hkv, page_size, d), seed_base + 2, dtype),
        "v_pages": seeded_normal((num_pages, Hkv, page_size, d), seed_base + 3, dtype),
        "block_table": torch.from_numpy(table),
        "seq_lens": torch.from_numpy(lens.astype(np.int32)),
    }


def paged_workload_inputs(w: Workload) -> dict:
    return paged_cache(w.B, w.Hq, w.Hkv, w.nq, w.N, w.d, w.page_size, w.seed_base, min_len=2048)


def local_global_layout(N: int, local: int, nglobal: int) -> torch.Tensor:
    """uint8 [nb, nb] over 64 x 64 blocks (nb = ceil(N/64)): query block i sees key
    blocks j with |i - j| < local (a local band) and the first ``nglobal`` key blocks."""
    nb = (N + 63) // 64
    i = torch.arange(nb)[:, None]
    j = torch.arange(nb)[None, :]
    return (((i - j).abs() < local) | (j < nglobal)).to(torch.uint8)


def random_layout(N: int, density: float, seed: int) -> torch.Tensor:
    """uint8 [nb, nb] with each block set independently with probability ``density``."""
    nb = (N + 63) // 64
    g = torch.Generator().manual_seed(int(seed))
    return (torch.rand(nb, nb, generator=g) < density).to(torch.uint8)


def workload_layout(w: Workload) -> torch.Tensor:
    return local_global_layout(w.N, *w.layout)
