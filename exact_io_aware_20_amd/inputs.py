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
==========================  ====  ===  ===  =====  ===  ======  =====  ===========

The long-context workload multiplies q and k by 8 before the cast (a power of two,
exact in bf16), so logits reach |x| ~ 500 and stress the running-max rescaling.
The decode workloads hold a cache of N = 65536 keys and values per KV head and
Nq = 1 (one new token) or Nq = 4 (four tokens checked at once) queries per query
head; q is [B, Hq, Nq, d] and k, v are [B, Hkv, N, d].  The window workload lets each
query see only keys within 2047 positions (with the causal rule: its 2048 most recent
tokens, itself included).
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
