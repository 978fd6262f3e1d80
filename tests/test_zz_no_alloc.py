"""fa_backward_noalloc (the backward for callers that cannot allocate) against
fa_backward's deterministic steps, through the C ABI: two calls in a row on one
device, the second smaller, so the second runs on scratch the first has filled.

The two paths run the same kernels on the same inputs; the only difference is where
the per-row workspace lives, so the gradients must agree bit for bit (stricter than
the 1e-2 relative-L2 bar of the bf16 path, which is also checked against the oracle
on the smaller call).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_20_amd import api, inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16)


def _case(B, Hq, Hkv, N, d, causal, seed):
    sys.__stderr__.write(f"\n[gpu-case] no-alloc backward {B}x{Hq}x{Hkv}x{N}x{d} causal={causal}\n")
    sys.__stderr__.flush()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    host = inputs.make_inputs(B, Hq, Hkv, N, d, seed, torch.bfloat16, with_do=True)
    g = {k: v.to(dev) for k, v in host.items()}
    scale = 1.0 / math.sqrt(d)
    o, lse = api.forward(g["q"], g["k"], g["v"], causal, scale)
    ref = tuple(torch.full_like(g[n], float("nan")) for n in ("q", "k", "v"))
    ws = torch.empty(api.workspace_bytes(B, Hq, N), dtype=torch.uint8, device=dev)
    api.backward_steps(g["q"], g["k"], g["v"], o, g["do"], lse, causal, scale, *ref, ws)
    got = tuple(torch.full_like(g[n], float("nan")) for n in ("q", "k", "v"))
    api.backward_noalloc(g["q"], g["k"], g["v"], o, g["do"], lse, causal, scale, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a).all(), name
        assert torch.equal(_bits(a), _bits(b)), name
    return host, got


def test_noalloc_matches_backward_two_calls_second_smaller():
    _case(2, 32, 8, 2048, 128, True, 12000)          # 131072 query rows
    host, got = _case(1, 4, 2, 333, 64, False, 12001)  # fewer rows: stale scratch beyond them
    refs = oracle.attention_backward(host["q"], host["k"], host["v"], host["do"], False, 1.0 / math.sqrt(64))
    for name, a, r in zip(("dq", "dk", "dv"), got, refs):
        a = a.detach().cpu().double().numpy()
        rel = np.linalg.norm((a - r).ravel()) / np.linalg.norm(r.ravel())
        assert rel <= 1e-2, (name, rel)


def test_noalloc_rejects_more_rows_than_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    B, Hq, Hkv, N, d = 1, 1, 1, (1 << 21) + 64, 64
    t = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((B, Hq, N), dtype=torch.float32, device=dev)
    with pytest.raises(api.FAError) as e:
        api.backward_noalloc(t, t.clone(), t.clone(), t.clone(), t.clone(), lse, True, 0.1)
    assert e.value.code == 12
