"""The C-ABI library loads, exports what include/fa.h declares, and validates
arguments on the host (no GPU needed: nothing here launches a kernel).

If the library has not been built, it is built here first (hipcc cross-compiles the
gfx950 code without a GPU), so these checks always run.  The same module also runs
against a host-only build of the ABI (fa_api.cpp and the launch plans, with counting
stand-ins for the launchers) made with AddressSanitizer and UndefinedBehaviorSanitizer
by tests/test_abi_host_asan.py; the tests marked ``stub_only`` need that build, since
they make calls that pass validation and would launch kernels in the real library.
"""
import ctypes
import math
import os
import re
from pathlib import Path

import pytest

from exact_io_aware_20_amd import api

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "fa.h"


@pytest.fixture(scope="module", autouse=True)
def _library():
    if not api.LIB_PATH.exists() and "FA_MI355X_LIB" not in os.environ:
        from exact_io_aware_20_amd.build import build_library
        build_library()
    assert api.LIB_PATH.exists(), api.LIB_PATH
    yield


def _is_stub() -> bool:
    return hasattr(api.load_library(), "fa_stub_launches")


def stub_only(fn):
    """Run only against the host-only sanitizer build (the calls pass validation)."""
    def wrapper(*a, **kw):
        if not _is_stub():
            pytest.skip("needs the host-only ABI build (tests/test_abi_host_asan.py runs it)")
        return fn(*a, **kw)
    wrapper.__name__ = fn.__name__
    return wrapper


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == sorted(api.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(api.LIB_PATH))
    assert not _is_stub() or os.environ.get("FA_MI355X_LIB")
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = api.load_library()
    for code, name in api.FA_STATUS.items():
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status", name
    assert lib.fa_status_string(99).decode() == "unknown status"


def test_workspace_bytes():
    lib = api.load_library()
    rows = 2 * 32 * 8192
    # D and LSE in base 2: 8 bytes per row
    assert lib.fa_backward_workspace_bytes(2, 32, 8192) == 8 * rows
    # the fused alternative: the same, then from a 256-byte boundary an fp32 dQ
    # accumulator of d values per row
    assert lib.fa_backward_fused_workspace_bytes(2, 32, 8192, 128) == 8 * rows + 512 * rows
    assert lib.fa_backward_fused_workspace_bytes(1, 1, 3, 64) == 256 + 256 * 3
    assert lib.fa_backward_fused_workspace_bytes(1, 1, 3, 96) == 0
    assert lib.fa_backward_workspace_bytes(0, 1, 1) == 0
    assert lib.fa_backward_workspace_bytes(1, 1, -5) == 0


# Fake, never-dereferenced device addresses, 1 GiB apart and 256-byte aligned.
Q, K, V, O, L = (0x10_0000_0000 + i * (1 << 30) for i in range(5))


def check(q=Q, k=K, v=V, o=O, lse=L, B=2, Hq=4, Hkv=2, N=100, d=64, causal=1, scale=0.125, elt=2):
    return api.load_library().fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, elt)


@pytest.mark.parametrize("kwargs,code", [
    ({}, 0),
    ({"elt": 4, "d": 128}, 0),
    ({"causal": 0}, 0),
    ({"scale": 0.0}, 0),
    ({"q": None}, 1), ({"k": None}, 1), ({"v": None}, 1), ({"o": None}, 1), ({"lse": None}, 1),
    ({"B": 0}, 2), ({"Hq": 0}, 2), ({"Hkv": 0}, 2), ({"N": 0}, 2), ({"N": -3}, 2), ({"elt": 3}, 2),
    ({"Hq": 6, "Hkv": 4}, 3),
    ({"d": 96}, 4), ({"d": 256}, 4), ({"d": 0}, 4),
    ({"scale": float("nan")}, 5), ({"scale": float("inf")}, 5), ({"scale": -1.0}, 5),
    ({"q": Q + 8}, 6), ({"o": O + 2}, 6), ({"lse": L + 4}, 6),
    ({"causal": 2}, 7), ({"causal": -1}, 7),
    ({"o": Q}, 9), ({"o": K + 64}, 9), ({"lse": O + 16}, 9), ({"lse": V}, 9),
    ({"B": 1 << 20, "Hq": 1 << 10, "Hkv": 1 << 10, "N": 1 << 16}, 2),
])
def test_check_args_codes(kwargs, code):
    assert check(**kwargs) == code


def test_forward_rejects_before_launch():
    # Invalid calls return their code without touching the GPU.
    lib = api.load_library()
    assert lib.fa_forward(None, K, V, O, L, 1, 1, 1, 8, 64, 0, 0.1, None) == 1
    assert lib.fa_forward(Q, K, V, O, L, 1, 1, 1, 8, 80, 0, 0.1, None) == 4
    assert lib.fa_forward_f32(Q, K, V, O, L, 1, 3, 2, 8, 64, 0, 0.1, None) == 3


def test_backward_rejects_before_launch():
    lib = api.load_library()
    base = [Q, K, V, O, 0x20_0000_0000, L, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000]
    ws = 0x60_0000_0000
    args = lambda ptrs, ws_, wsb, **kw: lib.fa_backward(
        *ptrs, ws_, wsb, kw.get("B", 1), kw.get("Hq", 2), kw.get("Hkv", 1), kw.get("N", 16),
        kw.get("d", 64), kw.get("causal", 1), kw.get("scale", 0.125), None)
    need = lib.fa_backward_workspace_bytes(1, 2, 16)
    assert args(base, None, need) == 8
    assert args(base, ws, need - 4) == 8
    assert args(base, ws + 4, need) == 8
    assert args([None] + base[1:], ws, need) == 1
    assert args(base, ws, need, d=32) == 4
    bad = list(base)
    bad[6] = base[0]  # dq aliases q
    assert args(bad, ws, need) == 9
    bad = list(base)
    bad[8] = base[7]  # dv aliases dk
    assert args(bad, ws, need) == 9
    assert args(base, base[0], need) == 9  # workspace aliases q


def test_backward_steps_reject_before_launch():
    lib = api.load_library()
    dO, lse, ws, dq, dk, dv = (0x20_0000_0000, L, 0x60_0000_0000, 0x30_0000_0000, 0x40_0000_0000,
                               0x50_0000_0000)
    need = lib.fa_backward_workspace_bytes(1, 2, 16)
    # preprocess reads o, dO and lse, writes the workspace (D and LSE in base 2)
    assert lib.fa_backward_preprocess(O, dO, None, ws, need, 1, 2, 16, 64, None) == 1
    assert lib.fa_backward_preprocess(O, dO, lse, ws, need - 4, 1, 2, 16, 64, None) == 8
    assert lib.fa_backward_preprocess(O, dO, lse, lse, need, 1, 2, 16, 64, None) == 9
    assert lib.fa_backward_preprocess(O, dO, lse, ws, need, 1, 2, 16, 48, None) == 4
    # dK/dV and dQ read q, k, v, dO and the workspace only
    assert lib.fa_backward_dkdv(Q, K, V, dO, None, need, dk, dv, 1, 2, 1, 16, 64, 1, 0.1, None) == 8
    assert lib.fa_backward_dkdv(Q, K, V, dO, ws, need, dk, dk, 1, 2, 1, 16, 64, 1, 0.1, None) == 9
    assert lib.fa_backward_dkdv(Q, K, V, dO, ws, need, dk, dv, 1, 2, 1, 16, 64, 2, 0.1, None) == 7
    assert lib.fa_backward_dq(Q, K, V, dO, ws, need, Q, 1, 2, 1, 16, 64, 1, 0.1, None) == 9
    assert lib.fa_backward_dq(Q, K, V, dO, ws, need, dq, 1, 3, 2, 16, 64, 1, 0.1, None) == 3
    # the preprocess and dQ in one kernel: reads o, dO, lse, q, k, v; writes the workspace and dq
    assert lib.fa_backward_preprocess_dq(Q, K, V, O, dO, None, ws, need, dq, 1, 2, 1, 16, 64, 1, 0.1, None) == 1
    assert lib.fa_backward_preprocess_dq(Q, K, V, O, dO, lse, ws, need - 4, dq, 1, 2, 1, 16, 64, 1, 0.1, None) == 8
    assert lib.fa_backward_preprocess_dq(Q, K, V, O, dO, lse, lse, need, dq, 1, 2, 1, 16, 64, 1, 0.1, None) == 9
    assert lib.fa_backward_preprocess_dq(Q, K, V, O, dO, lse, ws, need, O, 1, 2, 1, 16, 64, 1, 0.1, None) == 9
    assert lib.fa_backward_preprocess_dq(Q, K, V, O, dO, lse, ws, need, dq, 1, 3, 2, 16, 64, 1, 0.1, None) == 3


def test_decode_workspace_bytes():
    lib = api.load_library()
    # one fp32 row of d partial outputs plus one partial LSE per query row and key split
    for B, Hq, Hkv, Nq, Nk, d in ((8, 24, 2, 1, 65536, 128), (2, 8, 1, 5, 1000, 64), (1, 1, 1, 1, 1, 64),
                                  (4, 32, 8, 4, 32768, 128)):
        nb = lib.fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
        per_split = B * Hq * Nq * (d + 1) * 4
        assert nb > 0 and nb % per_split == 0
        assert 1 <= nb // per_split <= (Nk + 63) // 64
    assert lib.fa_decode_workspace_bytes(0, 1, 1, 1, 8, 64) == 0
    assert lib.fa_decode_workspace_bytes(1, 3, 2, 1, 8, 64) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 1, 0, 8, 64) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 1, 1, 8, 80) == 0


def test_decode_rejects_before_launch():
    lib = api.load_library()
    ws = 0x60_0000_0000
    args = lambda q=Q, o=O, lse=L, ws_=ws, wsb=None, **kw: lib.fa_decode_forward(
        q, K, V, o, lse, ws_,
        lib.fa_decode_workspace_bytes(kw.get("B", 1), kw.get("Hq", 4), kw.get("Hkv", 2), kw.get("Nq", 2),
                                      kw.get("Nk", 100), kw.get("d", 64)) if wsb is None else wsb,
        kw.get("B", 1), kw.get("Hq", 4), kw.get("Hkv", 2), kw.get("Nq", 2), kw.get("Nk", 100), kw.get("d", 64),
        kw.get("causal", 1), kw.get("scale", 0.125), None)
    assert args(q=None) == 1
    assert args(ws_=None) == 8
    assert args(wsb=16) == 8
    assert args(ws_=ws + 4) == 8
    assert args(Nq=0) == 2
    assert args(Nq=101) == 2          # causal: the queries must be the tail of the cache
    assert args(Hq=3) == 3
    assert args(d=96) == 4
    assert args(causal=2) == 7
    assert args(scale=float("nan")) == 5
    assert args(o=Q) == 9             # o aliases q
    assert args(ws_=K) == 9           # workspace aliases k


def test_decode_steps_reject_before_launch():
    lib = api.load_library()
    need = lib.fa_decode_workspace_bytes(1, 4, 2, 2, 100, 64)
    for fn in (lib.fa_decode_split, lib.fa_decode_merge):
        assert fn(Q, K, V, O, L, 0x60_0000_0000, need - 4, 1, 4, 2, 2, 100, 64, 1, 0.1, None) == 8
        assert fn(Q, K, V, O, O, 0x60_0000_0000, need, 1, 4, 2, 2, 100, 64, 1, 0.1, None) == 9
        assert fn(Q, K, V, O, L, 0x60_0000_0000, need, 1, 4, 2, 200, 100, 64, 1, 0.1, None) == 2


def test_window_calls_reject_before_launch():
    lib = api.load_library()
    dO, ws, dq, dk, dv = 0x20_0000_0000, 0x60_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000
    need = lib.fa_backward_workspace_bytes(1, 2, 16)
    assert lib.fa_forward_window(Q, K, V, O, L, 1, 2, 1, 16, 64, 1, -1, 0.1, None) == 11
    assert lib.fa_forward_window(Q, K, V, O, L, 1, 2, 1, 16, 80, 1, 4, 0.1, None) == 4
    assert lib.fa_forward_window(Q, K, V, Q, L, 1, 2, 1, 16, 64, 1, 4, 0.1, None) == 9
    assert lib.fa_backward_window(Q, K, V, O, dO, L, dq, dk, dv, ws, need, 1, 2, 1, 16, 64, 1, -3, 0.1, None) == 11
    assert lib.fa_backward_window(Q, K, V, O, dO, L, dq, dk, dv, ws, need - 4, 1, 2, 1, 16, 64, 1, 3, 0.1,
                                  None) == 8
    assert lib.fa_backward_dkdv_window(Q, K, V, dO, ws, need, dk, dv, 1, 2, 1, 16, 64, 1, -1, 0.1, None) == 11
    assert lib.fa_backward_dkdv_window(Q, K, V, dO, ws, need, dk, dk, 1, 2, 1, 16, 64, 1, 2, 0.1, None) == 9
    assert lib.fa_backward_dq_window(Q, K, V, dO, ws, need, dq, 1, 2, 1, 16, 64, 1, -1, 0.1, None) == 11
    assert lib.fa_backward_dq_window(Q, K, V, dO, ws, need, dq, 1, 3, 2, 16, 64, 1, 2, 0.1, None) == 3


def test_paged_decode_rejects_before_launch():
    lib = api.load_library()
    KP, VP, TB, SL, ws = 0x70_0000_0000, 0x71_0000_0000, 0x72_0000_0000, 0x73_0000_0000, 0x60_0000_0000
    need = lib.fa_decode_workspace_bytes(2, 4, 2, 1, 1000, 128)

    def call(q=Q, kp=KP, tb=TB, sl=SL, o=O, wsb=None, **kw):
        a = dict(B=2, Hq=4, Hkv=2, Nq=1, L=1000, P=10, psize=128, mb=8, d=128, causal=1)
        a.update(kw)
        return lib.fa_decode_paged_forward(q, kp, VP, tb, sl, o, L, ws, need if wsb is None else wsb, a["B"],
                                           a["Hq"], a["Hkv"], a["Nq"], a["L"], a["P"], a["psize"], a["mb"], a["d"],
                                           a["causal"], 0.1, None)
    assert call(tb=None) == 1
    assert call(psize=100) == 2          # not a multiple of 64
    assert call(mb=7) == 2               # 7 * 128 < 1000 tokens
    assert call(P=0) == 2
    assert call(tb=TB + 2) == 6          # int32 table needs 4-byte alignment
    assert call(wsb=need - 4) == 8
    assert call(o=KP) == 9               # o overlaps the K pool
    assert call(Nq=1001) == 2            # causal: more queries than the longest sequence


def test_blocksparse_calls_reject_before_launch():
    lib = api.load_library()
    dO, ws, dq, dk, dv, BM = (0x20_0000_0000, 0x60_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000,
                              0x80_0000_0000)
    need = lib.fa_backward_workspace_bytes(1, 2, 16)
    assert lib.fa_forward_blocksparse(Q, K, V, O, L, None, 1, 2, 1, 16, 64, 1, 0.1, None) == 1
    assert lib.fa_forward_blocksparse(Q, K, V, O, L, BM, 1, 2, 1, 200000, 64, 1, 0.1, None) == 2   # > 2048 blocks
    assert lib.fa_forward_blocksparse(Q, K, V, O, L, O, 1, 2, 1, 16, 64, 1, 0.1, None) == 9        # layout = o
    assert lib.fa_forward_blocksparse(Q, K, V, O, L, BM, 1, 2, 1, 16, 80, 1, 0.1, None) == 4
    assert lib.fa_backward_blocksparse(Q, K, V, O, dO, L, dq, dk, dv, None, ws, need, 1, 2, 1, 16, 64, 1, 0.1,
                                       None) == 1
    assert lib.fa_backward_blocksparse(Q, K, V, O, dO, L, dq, dk, dv, dq, ws, need, 1, 2, 1, 16, 64, 1, 0.1,
                                       None) == 9
    small = 8 * 2 * 16   # the dK/dV step reads only D and LSE in base 2
    assert lib.fa_backward_dkdv_blocksparse(Q, K, V, dO, ws, small - 4, dk, dv, BM, 1, 2, 1, 16, 64, 1, 0.1,
                                            None) == 8
    assert lib.fa_backward_dq_blocksparse(Q, K, V, dO, ws, need, dq, BM, 1, 3, 2, 16, 64, 1, 0.1, None) == 3


def test_blocksparse_layout_inside_workspace_is_an_alias_whatever_workspace_bytes_says():
    # The overlap test uses the workspace extent the call writes, not the caller's
    # figure: with SIZE_MAX the end address would wrap and hide the overlap.
    lib = api.load_library()
    dO, ws, dq, dk, dv = 0x20_0000_0000, 0x60_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000
    need = lib.fa_backward_workspace_bytes(1, 2, 16)
    huge = (1 << 64) - 1
    inside = ws + 64
    assert lib.fa_backward_blocksparse(Q, K, V, O, dO, L, dq, dk, dv, inside, ws, huge, 1, 2, 1, 16, 64, 1, 0.1,
                                       None) == 9
    assert lib.fa_backward_blocksparse(Q, K, V, O, dO, L, dq, dk, dv, inside, ws, need, 1, 2, 1, 16, 64, 1, 0.1,
                                       None) == 9


# ---------------------------------------------------------------- host-only build: calls that pass

def _launches():
    return api.load_library().fa_stub_launches()


@stub_only
def test_every_entry_point_launches_only_after_validation():
    lib = api.load_library()
    lib.fa_stub_launches.restype = ctypes.c_longlong
    dO, ws, dq, dk, dv, BM = (0x20_0000_0000, 0x60_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000,
                              0x80_0000_0000)
    KP, VP, TB, SL = 0x70_0000_0000, 0x71_0000_0000, 0x72_0000_0000, 0x73_0000_0000
    need = lib.fa_backward_workspace_bytes(2, 4, 300)
    fneed = lib.fa_backward_fused_workspace_bytes(2, 4, 300, 128)
    dneed = lib.fa_decode_workspace_bytes(2, 4, 2, 3, 1000, 128)
    # (name, launcher calls when valid (decode: one call covers its split and merge),
    #  valid call, a rejected variant)
    calls = [
        ("fa_forward", 1, lambda c: lib.fa_forward(Q, K, V, O, L, 2, 4, 2, 300, 128, c, 0.1, None),
         lambda: lib.fa_forward(Q, K, V, O, L, 2, 4, 2, 300, 96, 1, 0.1, None)),
        ("fa_forward_fp32_out", 1, lambda c: lib.fa_forward_fp32_out(Q, K, V, O, L, 2, 4, 2, 300, 128, c, 0.1,
                                                                      None),
         lambda: lib.fa_forward_fp32_out(Q, K, V, L - 64, L, 2, 4, 2, 300, 128, 1, 0.1, None)),
        ("fa_forward_f32", 1, lambda c: lib.fa_forward_f32(Q, K, V, O, L, 2, 4, 2, 300, 64, c, 0.1, None),
         lambda: lib.fa_forward_f32(Q, K, V, Q, L, 2, 4, 2, 300, 64, 1, 0.1, None)),
        ("fa_backward", 2, lambda c: lib.fa_backward(Q, K, V, O, dO, L, dq, dk, dv, ws, need, 2, 4, 2, 300, 128, c,
                                                      0.1, None),
         lambda: lib.fa_backward(Q, K, V, O, dO, L, dq, dk, dv, ws, need - 1, 2, 4, 2, 300, 128, 1, 0.1, None)),
        ("fa_backward_noalloc", 2, lambda c: lib.fa_backward_noalloc(Q, K, V, O, dO, L, dq, dk, dv, 2, 4, 2, 300,
                                                                      128, c, 0.1, None),
         lambda: lib.fa_backward_noalloc(Q, K, V, O, dO, L, dq, dk, dv, 8, 32, 32, 8193, 128, 1, 0.1, None)),
        ("fa_backward_preprocess", 1, lambda c: lib.fa_backward_preprocess(O, dO, L, ws, need, 2, 4, 300, 128, None),
         lambda: lib.fa_backward_preprocess(O, dO, L, O, need, 2, 4, 300, 128, None)),
        ("fa_backward_dkdv", 1, lambda c: lib.fa_backward_dkdv(Q, K, V, dO, ws, need, dk, dv, 2, 4, 2, 300, 64, c,
                                                                0.1, None),
         lambda: lib.fa_backward_dkdv(Q, K, V, dO, ws, need, dk, K, 2, 4, 2, 300, 64, 1, 0.1, None)),
        ("fa_backward_dq", 1, lambda c: lib.fa_backward_dq(Q, K, V, dO, ws, need, dq, 2, 4, 2, 300, 64, c, 0.1,
                                                            None),
         lambda: lib.fa_backward_dq(Q, K, V, dO, ws, need, dq, 2, 4, 3, 300, 64, 1, 0.1, None)),
        ("fa_backward_preprocess_dq", 1,
         lambda c: lib.fa_backward_preprocess_dq(Q, K, V, O, dO, L, ws, need, dq, 2, 4, 2, 300, 128, c, 0.1, None),
         lambda: lib.fa_backward_preprocess_dq(Q, K, V, O, dO, L, ws, need, dq, 2, 4, 3, 300, 128, 1, 0.1, None)),
        ("fa_backward_fused", 3, lambda c: lib.fa_backward_fused(Q, K, V, O, dO, L, dq, dk, dv, ws, fneed, 2, 4, 2,
                                                                  300, 128, c, 0.1, None),
         lambda: lib.fa_backward_fused(Q, K, V, O, dO, L, dq, dk, dv, ws, need, 2, 4, 2, 300, 128, 1, 0.1, None)),
        ("fa_backward_dkdv_dq", 1, lambda c: lib.fa_backward_dkdv_dq(Q, K, V, dO, ws, fneed, dk, dv, 2, 4, 2, 300,
                                                                      128, c, 0.1, None),
         lambda: lib.fa_backward_dkdv_dq(Q, K, V, dO, ws, need, dk, dv, 2, 4, 2, 300, 128, 1, 0.1, None)),
        ("fa_backward_dq_convert", 1, lambda c: lib.fa_backward_dq_convert(ws, fneed, dq, 2, 4, 300, 128, 0.1, None),
         lambda: lib.fa_backward_dq_convert(ws, fneed, ws + 64, 2, 4, 300, 128, 0.1, None)),
        ("fa_forward_window", 1, lambda c: lib.fa_forward_window(Q, K, V, O, L, 2, 4, 2, 300, 128, c, 17, 0.1,
                                                                  None),
         lambda: lib.fa_forward_window(Q, K, V, O, L, 2, 4, 2, 300, 128, 1, -2, 0.1, None)),
        ("fa_backward_window", 2, lambda c: lib.fa_backward_window(Q, K, V, O, dO, L, dq, dk, dv, ws, need, 2, 4, 2,
                                                                    300, 128, c, 17, 0.1, None),
         lambda: lib.fa_backward_window(Q, K, V, O, dO, L, dq, dk, dv, ws, need, 2, 4, 2, 300, 128, 1, 17,
                                        float("inf"), None)),
        ("fa_backward_dkdv_window", 1, lambda c: lib.fa_backward_dkdv_window(Q, K, V, dO, ws, need, dk, dv, 2, 4, 2,
                                                                              300, 64, c, 5, 0.1, None),
         lambda: lib.fa_backward_dkdv_window(Q, K, V, dO, ws, need, dk, dv, 2, 4, 2, 300, 64, 1, -1, 0.1, None)),
        ("fa_backward_dq_window", 1, lambda c: lib.fa_backward_dq_window(Q, K, V, dO, ws, need, dq, 2, 4, 2, 300,
                                                                          64, c, 5, 0.1, None),
         lambda: lib.fa_backward_dq_window(Q, K, V, dO, None, need, dq, 2, 4, 2, 300, 64, 1, 5, 0.1, None)),
        ("fa_backward_preprocess_dq_window", 1,
         lambda c: lib.fa_backward_preprocess_dq_window(Q, K, V, O, dO, L, ws, need, dq, 2, 4, 2, 300, 64, c, 5, 0.1,
                                                        None),
         lambda: lib.fa_backward_preprocess_dq_window(Q, K, V, O, dO, L, ws, need, dq, 2, 4, 2, 300, 64, 1, -1, 0.1,
                                                      None)),
        ("fa_forward_blocksparse", 1, lambda c: lib.fa_forward_blocksparse(Q, K, V, O, L, BM, 2, 4, 2, 300, 128, c,
                                                                            0.1, None),
         lambda: lib.fa_forward_blocksparse(Q, K, V, O, L, L, 2, 4, 2, 300, 128, 1, 0.1, None)),
        ("fa_backward_blocksparse", 3, lambda c: lib.fa_backward_blocksparse(Q, K, V, O, dO, L, dq, dk, dv, BM, ws,
                                                                              need, 2, 4, 2, 300, 128, c, 0.1, None),
         lambda: lib.fa_backward_blocksparse(Q, K, V, O, dO, L, dq, dk, dv, dk, ws, need, 2, 4, 2, 300, 128, 1,
                                             0.1, None)),
        ("fa_backward_dkdv_blocksparse", 1,
         lambda c: lib.fa_backward_dkdv_blocksparse(Q, K, V, dO, ws, need, dk, dv, BM, 2, 4, 2, 300, 64, c, 0.1,
                                                    None),
         lambda: lib.fa_backward_dkdv_blocksparse(Q, K, V, dO, ws, need, dk, dv, None, 2, 4, 2, 300, 64, 1, 0.1,
                                                  None)),
        ("fa_backward_dq_blocksparse", 1,
         lambda c: lib.fa_backward_dq_blocksparse(Q, K, V, dO, ws, need, dq, BM, 2, 4, 2, 300, 64, c, 0.1, None),
         lambda: lib.fa_backward_dq_blocksparse(Q, K, V, dO, ws, need, dq, BM, 2, 4, 2, 300, 64, 5, 0.1, None)),
        ("fa_backward_preprocess_dq_blocksparse", 1,
         lambda c: lib.fa_backward_preprocess_dq_blocksparse(Q, K, V, O, dO, L, ws, need, dq, BM, 2, 4, 2, 300, 64, c,
                                                             0.1, None),
         lambda: lib.fa_backward_preprocess_dq_blocksparse(Q, K, V, O, dO, L, ws, need, dq, None, 2, 4, 2, 300, 64, 1,
                                                           0.1, None)),
        ("fa_decode_forward", 1, lambda c: lib.fa_decode_forward(Q, K, V, O, L, ws, dneed, 2, 4, 2, 3, 1000, 128, c,
                                                                  0.1, None),
         lambda: lib.fa_decode_forward(Q, K, V, O, L, ws, dneed - 1, 2, 4, 2, 3, 1000, 128, 1, 0.1, None)),
        ("fa_decode_split", 1, lambda c: lib.fa_decode_split(Q, K, V, O, L, ws, dneed, 2, 4, 2, 3, 1000, 128, c,
                                                              0.1, None),
         lambda: lib.fa_decode_split(Q, K, V, O, L, ws, dneed, 2, 4, 2, 1001, 1000, 128, 1, 0.1, None)),
        ("fa_decode_merge", 1, lambda c: lib.fa_decode_merge(Q, K, V, O, L, ws, dneed, 2, 4, 2, 3, 1000, 128, c,
                                                              0.1, None),
         lambda: lib.fa_decode_merge(Q, K, V, O, L, K, dneed, 2, 4, 2, 3, 1000, 128, 1, 0.1, None)),
        ("fa_decode_paged_forward", 1,
         lambda c: lib.fa_decode_paged_forward(Q, KP, VP, TB, SL, O, L, ws, dneed, 2, 4, 2, 3, 1000, 10, 128, 8,
                                               128, c, 0.1, None),
         lambda: lib.fa_decode_paged_forward(Q, KP, VP, TB, SL, O, L, ws, dneed, 2, 4, 2, 3, 1000, 10, 100, 8,
                                             128, 1, 0.1, None)),
        ("fa_decode_paged_split", 1,
         lambda c: lib.fa_decode_paged_split(Q, KP, VP, TB, SL, O, L, ws, dneed, 2, 4, 2, 3, 1000, 10, 128, 8,
                                             128, c, 0.1, None),
         lambda: lib.fa_decode_paged_split(Q, KP, VP, TB + 1, SL, O, L, ws, dneed, 2, 4, 2, 3, 1000, 10, 128, 8,
                                           128, 1, 0.1, None)),
        ("fa_decode_paged_merge", 1,
         lambda c: lib.fa_decode_paged_merge(Q, KP, VP, TB, SL, O, L, ws, dneed, 2, 4, 2, 3, 1000, 10, 128, 8,
                                             128, c, 0.1, None),
         lambda: lib.fa_decode_paged_merge(Q, KP, VP, TB, SL, O, L, ws, dneed, 2, 4, 2, 3, 1000, 10, 128, 7,
                                           128, 1, 0.1, None)),
    ]
    named = {c[0] for c in calls}
    computing = {n for n in declared_functions()
                 if n not in ("fa_backward_workspace_bytes", "fa_decode_workspace_bytes", "fa_check_args",
                              "fa_status_string", "fa_backward_fused_workspace_bytes")}
    assert computing <= named, sorted(computing - named)
    for name, n_launch, ok, bad in calls:
        for causal in (0, 1):
            before = _launches()
            assert ok(causal) == 0, name
            assert _launches() - before == n_launch, name
        before = _launches()
        assert bad() != 0, name
        assert _launches() == before, name


def test_noalloc_backward_rejects_before_launch():
    lib = api.load_library()
    dO, dq, dk, dv = 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000
    call = lambda *ptrs, B=1, Hq=2, Hkv=1, N=16, d=64, causal=1, scale=0.1: lib.fa_backward_noalloc(
        *ptrs, B, Hq, Hkv, N, d, causal, scale, None)
    base = (Q, K, V, O, dO, L, dq, dk, dv)
    assert call(*base, N=(1 << 21) // 2 + 1) == 12          # 2^21 + 2 query rows: over the scratch
    assert call(*base, B=8, Hq=32, Hkv=8, N=8193) == 12     # 2^21 rows fit, 256 more do not
    assert call(None, *base[1:]) == 1
    assert call(*base, d=96) == 4
    assert call(*base[:6], Q, dk, dv) == 9                  # dq aliases q
    assert call(*base, scale=float("nan")) == 5
    assert lib.fa_status_string(12).decode().startswith("B * Hq * N exceeds")


def test_fused_steps_need_the_accumulator():
    lib = api.load_library()
    dO, ws, dq, dk, dv = 0x20_0000_0000, 0x60_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000
    small = lib.fa_backward_workspace_bytes(1, 2, 16)
    full = lib.fa_backward_fused_workspace_bytes(1, 2, 16, 64)
    # the fused steps and the fused whole call need the accumulator after the per-row terms
    assert lib.fa_backward_fused(Q, K, V, O, dO, L, dq, dk, dv, ws, full - 1, 1, 2, 1, 16, 64, 1, 0.1, None) == 8
    assert lib.fa_backward_dkdv_dq(Q, K, V, dO, ws, small, dk, dv, 1, 2, 1, 16, 64, 1, 0.1, None) == 8
    assert lib.fa_backward_dkdv_dq(Q, K, V, dO, ws, full - 1, dk, dv, 1, 2, 1, 16, 64, 1, 0.1, None) == 8
    assert lib.fa_backward_dq_convert(ws, full - 1, dq, 1, 2, 16, 64, 0.1, None) == 8
    assert lib.fa_backward_dq_convert(ws, full, None, 1, 2, 16, 64, 0.1, None) == 1
    assert lib.fa_backward_dq_convert(ws, full, dq, 1, 2, 16, 64, float("nan"), None) == 5
    # the fused kernel writes the accumulator: it may not overlap an input
    assert lib.fa_backward_dkdv_dq(Q, K, V, dO, Q - 64, full, dk, dv, 1, 2, 1, 16, 64, 1, 0.1, None) == 9
