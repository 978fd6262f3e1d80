"""Parity of the sliding-window path (fa_forward_window / fa_backward_window, through
the C ABI) with the CPU float64 oracle's window mask: key j visible to query i only
if |i - j| <= window (and j <= i when causal).

Bars (as for the full-sequence bf16 path): |O - O_ref| <= 1e-2 + half a bf16 ulp,
|LSE - LSE_ref| <= 1e-2, relative L2 <= 1e-2 for dQ, dK and dV.  Small shapes cover
windows of 0 and 1, windows at and around the tile sizes, windows wider than the
sequence, ragged tails, grouped-query heads, both head sizes and both mask settings;
the window workload is checked at full size on sampled rows and two KV groups.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_20_amd import api, inputs
from tests.test_parity_gpu import WORKERS, assert_o_bf16, dev, f64, make, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


FWD = [  # (B, Hq, Hkv, N, d, window)
    (1, 1, 1, 1, 64, 0), (1, 2, 1, 65, 128, 0), (1, 2, 1, 65, 64, 1), (2, 4, 2, 300, 128, 63),
    (1, 2, 2, 300, 64, 64), (1, 3, 1, 513, 128, 100), (1, 2, 1, 1000, 64, 255), (1, 4, 2, 1000, 128, 300),
    (1, 2, 1, 777, 128, 775), (1, 1, 1, 600, 64, 2000), (1, 2, 1, 2048, 128, 511),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", FWD, ids=lambda s: "x".join(map(str, s)))
def test_window_forward_small(shape, causal):
    B, Hq, Hkv, N, d, window = shape
    host, g = make(B, Hq, Hkv, N, d, seed=13000 + N + window)
    scale = 1.0 / math.sqrt(d)
    o, lse = api.forward(g["q"], g["k"], g["v"], causal, scale, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(host["q"], host["k"], host["v"], causal, scale, window=window)
    err = assert_o_bf16(f64(o), o_ref, str(shape))
    lerr = float(np.abs(f64(lse) - lse_ref).max())
    print(f"[parity] window fwd {shape} causal={causal} O {err:.3e} LSE {lerr:.3e}")
    assert lerr <= 1e-2


BWD = [(1, 2, 1, 65, 64, 1), (2, 4, 2, 300, 128, 63), (1, 3, 1, 513, 128, 100), (1, 4, 2, 1000, 128, 300),
       (1, 2, 1, 700, 64, 255), (1, 2, 2, 129, 64, 0)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", BWD, ids=lambda s: "x".join(map(str, s)))
def test_window_backward_small(shape, causal):
    B, Hq, Hkv, N, d, window = shape
    host, g = make(B, Hq, Hkv, N, d, seed=14000 + N + window, with_do=True)
    scale = 1.0 / math.sqrt(d)
    o, lse = api.forward(g["q"], g["k"], g["v"], causal, scale, window=window)
    dq, dk, dv = api.backward(g["q"], g["k"], g["v"], o, g["do"], lse, causal, scale, window=window)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(host["q"], host["k"], host["v"], host["do"], causal, scale, window=window)
    # With window 0 every softmax has one term, so dQ = dK = 0 exactly and a relative
    # error is undefined: an all-zero reference is checked by max-abs instead.
    errs = {n: (rel_l2(f64(a), r) if np.abs(r).max() > 0 else float(np.abs(f64(a)).max()))
            for n, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref)}
    print(f"[parity] window bwd {shape} causal={causal} " + " ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert max(errs.values()) <= 1e-2


def test_window_backward_steps_match_fused_call():
    B, Hq, Hkv, N, d, window = 1, 4, 2, 700, 128, 200
    host, g = make(B, Hq, Hkv, N, d, seed=14900, with_do=True)
    o, lse = api.forward(g["q"], g["k"], g["v"], True, 0.09, window=window)
    dq, dk, dv = api.backward(g["q"], g["k"], g["v"], o, g["do"], lse, True, 0.09, window=window)
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ws = torch.empty(api.workspace_bytes(B, Hq, N), dtype=torch.uint8, device=dev())
    api.backward_steps(g["q"], g["k"], g["v"], o, g["do"], lse, True, 0.09, dq2, dk2, dv2, ws, window=window)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_window_wider_than_sequence_matches_plain_call():
    # a window of N - 1 or more restricts nothing: bit-identical to fa_forward / fa_backward
    B, Hq, Hkv, N, d = 1, 2, 1, 400, 128
    host, g = make(B, Hq, Hkv, N, d, seed=14950, with_do=True)
    o1, l1 = api.forward(g["q"], g["k"], g["v"], True, 0.1)
    o2, l2 = api.forward(g["q"], g["k"], g["v"], True, 0.1, window=N - 1)
    g1 = api.backward(g["q"], g["k"], g["v"], o1, g["do"], l1, True, 0.1)
    g2 = api.backward(g["q"], g["k"], g["v"], o1, g["do"], l1, True, 0.1, window=5 * N)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_window_workload_full_size():
    w = inputs.WORKLOADS["window_n16384_w2047_d128"]
    host = inputs.workload_inputs(w)
    g = {k: v.to(dev()) for k, v in host.items()}
    o, lse = api.forward(g["q"], g["k"], g["v"], True, w.scale, window=w.window)
    dq, dk, dv = api.backward(g["q"], g["k"], g["v"], o, g["do"], lse, True, w.scale, window=w.window)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(dq).any()
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(w.N - 256, w.N),
                                     rng.choice(w.N, 1024, replace=False)]))
    heads = [(0, 0), (0, 9), (1, 5), (1, 15)]
    o_ref, lse_ref = oracle.attention_forward(host["q"], host["k"], host["v"], True, w.scale, heads=heads,
                                              rows=rows, workers=WORKERS, window=w.window)
    o_h, lse_h = f64(o), f64(lse)
    for b, h in heads:
        assert_o_bf16(o_h[b, h, rows], o_ref[b, h, rows], f"head {(b, h)}")
        assert np.abs(lse_h[b, h, rows] - lse_ref[b, h, rows]).max() <= 1e-2
    o_err = max(np.abs(o_h[b, h, rows] - o_ref[b, h, rows]).max() for b, h in heads)
    groups = [(0, 3), (1, 12)]
    dq_r, dk_r, dv_r = oracle.attention_backward(host["q"], host["k"], host["v"], host["do"], True, w.scale,
                                                 groups=groups, workers=WORKERS, window=w.window)
    e = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, hk in groups:
        e["dq"] = max(e["dq"], rel_l2(f64(dq[b, hk]), dq_r[b, hk]))
        e["dk"] = max(e["dk"], rel_l2(f64(dk[b, hk]), dk_r[b, hk]))
        e["dv"] = max(e["dv"], rel_l2(f64(dv[b, hk]), dv_r[b, hk]))
    print(f"\n[parity] window_n16384_w2047_d128: O max-abs {o_err:.3g} over {len(heads)} heads x {len(rows)} rows; "
          f"rel-L2 dQ {e['dq']:.3g} dK {e['dk']:.3g} dV {e['dv']:.3g}")
    assert max(e.values()) <= 1e-2
