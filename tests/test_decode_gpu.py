"""Parity of the decode path (fa_decode_forward, through the C ABI) with the CPU
float64 oracle's decode form: Nq new queries at the end of an Nk-token key/value
cache.

Bars (the same as the full-sequence bf16 forward, element by element):
|O - O_ref| <= 1e-2 + half a bf16 ulp of O_ref and |LSE - LSE_ref| <= 1e-2.
Small shapes cover caches shorter than one tile, ragged tails, one and several key
splits, one to four 32-row blocks of packed (head, query) rows, both head sizes and
both mask settings; the two decode workloads are checked whole at full size, and a
2^20-token cache (about a thousand splits merged per row) whole.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_20_amd import api, inputs
from tests.test_parity_gpu import WORKERS, assert_o_bf16, dev, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def make(B, Hq, Hkv, Nq, Nk, d, seed):
    host = inputs.make_inputs(B, Hq, Hkv, Nk, d, seed, torch.bfloat16, nq=Nq)
    return host, {k: v.to(dev()) for k, v in host.items()}


DEC_SMALL = [  # (B, Hq, Hkv, Nq, Nk, d)
    (1, 1, 1, 1, 1, 64), (1, 2, 1, 1, 63, 128), (1, 4, 4, 3, 64, 128), (2, 6, 2, 7, 129, 64),
    (1, 2, 2, 16, 16, 128), (2, 24, 2, 1, 1000, 128), (2, 24, 2, 4, 1000, 128), (1, 8, 1, 5, 300, 64),
    (1, 32, 1, 1, 4097, 128), (1, 3, 1, 40, 2000, 64), (3, 12, 4, 2, 20000, 128),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", DEC_SMALL, ids=lambda s: "x".join(map(str, s)))
def test_decode_small(shape, causal):
    B, Hq, Hkv, Nq, Nk, d = shape
    host, g = make(*shape, seed=11000 + Nk + Nq + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = api.decode_forward(g["q"], g["k"], g["v"], causal, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_forward(host["q"], host["k"], host["v"], causal, scale)
    err = assert_o_bf16(f64(o), o_ref, str(shape))
    lerr = float(np.abs(f64(lse) - lse_ref).max())
    print(f"[parity] decode {shape} causal={causal} O max-abs {err:.3e} LSE max-abs {lerr:.3e}")
    assert lerr <= 1e-2


def test_decode_more_queries_than_keys_without_mask():
    shape = (1, 4, 2, 70, 50, 64)
    host, g = make(*shape, seed=12001)
    o, lse = api.decode_forward(g["q"], g["k"], g["v"], False, 0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_forward(host["q"], host["k"], host["v"], False, 0.125)
    assert_o_bf16(f64(o), o_ref, str(shape))
    assert np.abs(f64(lse) - lse_ref).max() <= 1e-2


def test_decode_steps_match_fused_call():
    # split then merge through their own entry points gives the fused call's bits
    shape = (2, 24, 2, 4, 3000, 128)
    _, g = make(*shape, seed=12002)
    o1, l1 = api.decode_forward(g["q"], g["k"], g["v"], True, 0.09)
    ws = torch.empty(api.decode_workspace_bytes(*shape), dtype=torch.uint8, device=dev())
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    api.decode_forward(g["q"], g["k"], g["v"], True, 0.09, o=o2, lse=l2, workspace=ws, step="split")
    api.decode_forward(g["q"], g["k"], g["v"], True, 0.09, o=o2, lse=l2, workspace=ws, step="merge")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_with_whole_sequence_matches_forward_kernel():
    # Nq = Nk is the full-sequence forward: both kernels against the oracle, and
    # against each other within the bf16 bar.
    shape = (1, 4, 2, 300, 300, 128)
    host, g = make(*shape, seed=12003)
    scale = 1.0 / math.sqrt(128)
    od, ld = api.decode_forward(g["q"], g["k"], g["v"], True, scale)
    of, lf = api.forward(g["q"], g["k"], g["v"], True, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(host["q"], host["k"], host["v"], True, scale)
    assert_o_bf16(f64(od), o_ref, "decode")
    assert_o_bf16(f64(of), o_ref, "forward")
    assert np.abs(f64(ld) - lse_ref).max() <= 1e-2


def test_decode_reused_workspace_two_calls():
    # a second, smaller call on the same workspace and outputs' memory sees nothing
    # of the first
    big, small = (2, 24, 2, 4, 5000, 128), (1, 24, 2, 1, 700, 128)
    ws = torch.empty(api.decode_workspace_bytes(*big), dtype=torch.uint8, device=dev())
    for shape, seed in ((big, 12004), (small, 12005)):
        host, g = make(*shape, seed=seed)
        o, lse = api.decode_forward(g["q"], g["k"], g["v"], True, 0.1, workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.decode_forward(host["q"], host["k"], host["v"], True, 0.1)
        assert_o_bf16(f64(o), o_ref, str(shape))
        assert np.abs(f64(lse) - lse_ref).max() <= 1e-2


@pytest.mark.parametrize("name", ["decode_gqa_kv65536_d128", "decode_spec4_kv65536_d128"])
def test_decode_workload_full_size(name):
    # the benchmark's workload and launch configuration, every output row checked
    w = inputs.WORKLOADS[name]
    host = inputs.workload_inputs(w)
    g = {k: v.to(dev()) for k, v in host.items()}
    o, lse = api.decode_forward(g["q"], g["k"], g["v"], True, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_forward(host["q"], host["k"], host["v"], True, w.scale, workers=WORKERS)
    err = assert_o_bf16(f64(o), o_ref, name)
    lerr = float(np.abs(f64(lse) - lse_ref).max())
    print(f"[parity] {name} O max-abs {err:.3e} LSE max-abs {lerr:.3e}")
    assert lerr <= 1e-2


def test_decode_million_token_cache():
    # one sequence of 2^20 cached tokens: about 1024 key splits merged per row
    shape = (1, 8, 1, 2, 1 << 20, 128)
    host, g = make(*shape, seed=12100)
    o, lse = api.decode_forward(g["q"], g["k"], g["v"], True, 0.088)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_forward(host["q"], host["k"], host["v"], True, 0.088)
    err = assert_o_bf16(f64(o), o_ref, "1M cache")
    lerr = float(np.abs(f64(lse) - lse_ref).max())
    print(f"[parity] decode 2^20-token cache: O max-abs {err:.3e} LSE max-abs {lerr:.3e}")
    assert lerr <= 1e-2
