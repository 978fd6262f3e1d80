"""Python binding of libfa_mi355x.so (ctypes): argument marshalling only.

torch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

LIB_PATH = Path(os.environ.get("FA_MI355X_LIB", Path(__file__).resolve().parent / "libfa_mi355x.so"))

FA_STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_GQA", 4: "FA_ERR_HEADDIM",
    5: "FA_ERR_SCALE", 6: "FA_ERR_ALIGN", 7: "FA_ERR_FLAG", 8: "FA_ERR_WORKSPACE",
    9: "FA_ERR_ALIAS", 10: "FA_ERR_LAUNCH", 11: "FA_ERR_WINDOW", 12: "FA_ERR_SCRATCH",
}
ENTRY_POINTS = ("fa_forward", "fa_forward_f32", "fa_forward_fp32_out", "fa_backward", "fa_backward_workspace_bytes",
                "fa_backward_noalloc",
                "fa_backward_preprocess", "fa_backward_dkdv", "fa_backward_dq", "fa_backward_preprocess_dq",
                "fa_backward_dkdv_dq",
                "fa_backward_dq_convert", "fa_backward_fused", "fa_backward_fused_workspace_bytes",
                "fa_decode_forward", "fa_decode_workspace_bytes", "fa_decode_split", "fa_decode_merge",
                "fa_forward_window", "fa_backward_window", "fa_backward_dkdv_window", "fa_backward_dq_window",
                "fa_backward_preprocess_dq_window",
                "fa_decode_paged_forward", "fa_decode_paged_split", "fa_decode_paged_merge",
                "fa_forward_blocksparse", "fa_backward_blocksparse", "fa_backward_dkdv_blocksparse",
                "fa_backward_dq_blocksparse", "fa_backward_preprocess_dq_blocksparse",
                "fa_check_args", "fa_status_string")

_lib = None


class FAError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {FA_STATUS.get(code, code)}: {msg}")
        self.code = code


def load_library() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise FileNotFoundError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_20_amd.build`")
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_forward_f32.restype = i
    lib.fa_forward_fp32_out.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_forward_fp32_out.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_backward_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, vp]
    lib.fa_backward_preprocess.restype = i
    lib.fa_backward_dkdv.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dkdv.restype = i
    lib.fa_backward_dq.argtypes = [vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dq.restype = i
    lib.fa_backward_preprocess_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_preprocess_dq.restype = i
    lib.fa_backward_dkdv_dq.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dkdv_dq.restype = i
    lib.fa_backward_fused.argtypes = lib.fa_backward.argtypes
    lib.fa_backward_fused.restype = i
    lib.fa_backward_fused_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_backward_fused_workspace_bytes.restype = sz
    lib.fa_backward_dq_convert.argtypes = [vp, sz, vp, i, i, i, i, f, vp]
    lib.fa_backward_dq_convert.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i, i, i]
    lib.fa_backward_workspace_bytes.restype = sz
    lib.fa_decode_forward.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
    lib.fa_decode_forward.restype = i
    for fn in (lib.fa_decode_split, lib.fa_decode_merge):
        fn.argtypes = lib.fa_decode_forward.argtypes
        fn.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_forward_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_forward_window.restype = i
    lib.fa_backward_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
    lib.fa_backward_window.restype = i
    lib.fa_backward_dkdv_window.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dkdv_window.restype = i
    lib.fa_backward_dq_window.argtypes = [vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dq_window.restype = i
    lib.fa_backward_preprocess_dq_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_backward_preprocess_dq_window.restype = i
    for fn in (lib.fa_decode_paged_forward, lib.fa_decode_paged_split, lib.fa_decode_paged_merge):
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, i, i, i, f, vp]
        fn.restype = i
    lib.fa_forward_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_forward_blocksparse.restype = i
    lib.fa_backward_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    lib.fa_backward_blocksparse.restype = i
    lib.fa_backward_dkdv_blocksparse.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dkdv_blocksparse.restype = i
    lib.fa_backward_dq_blocksparse.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_backward_dq_blocksparse.restype = i
    lib.fa_backward_preprocess_dq_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, i, f,
                                                          vp]
    lib.fa_backward_preprocess_dq_blocksparse.restype = i
    lib.fa_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i]
    lib.fa_check_args.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().fa_status_string(code).decode()


def _check(fn: str, code: int):
    if code != 0:
        raise FAError(fn, code, status_string(code))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _shape(q: torch.Tensor, k: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    return B, Hq, k.shape[1], N, d


def _require(t: torch.Tensor, name: str, dtype, shape):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device} contiguous={t.is_contiguous()}")


def forward(q, k, v, causal: bool, scale: float, o=None, lse=None, stream=None, window=None, block_mask=None):
    """bf16 forward via fa_forward (or fa_forward_window when ``window`` is given, or
    fa_forward_blocksparse with a uint8 CUDA ``block_mask`` [nb, nb] over 64 x 64 blocks).
    Returns (o, lse); o bf16 [B,Hq,N,d], lse fp32 [B,Hq,N]."""
    if block_mask is not None:
        return _forward("fa_forward_blocksparse", torch.bfloat16, q, k, v, causal, scale, o, lse, stream,
                        layout=_layout(block_mask, q.shape[2], q.device))
    if window is not None:
        return _forward("fa_forward_window", torch.bfloat16, q, k, v, causal, scale, o, lse, stream, window)
    return _forward("fa_forward", torch.bfloat16, q, k, v, causal, scale, o, lse, stream)


def forward_fp32_out(q, k, v, causal: bool, scale: float, o=None, lse=None, stream=None):
    """Validation diagnostic via fa_forward_fp32_out: bf16 q, k, v; O returned in fp32
    as the bf16 kernel computes it before its final rounding.  Returns (o, lse)."""
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k)
    _require(q, "q", torch.bfloat16, (B, Hq, N, d))
    _require(k, "k", torch.bfloat16, (B, Hkv, N, d))
    _require(v, "v", torch.bfloat16, (B, Hkv, N, d))
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device) if o is None else o
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o, "o", torch.float32, (B, Hq, N, d))
    _require(lse, "lse", torch.float32, (B, Hq, N))
    code = lib.fa_forward_fp32_out(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   B, Hq, Hkv, N, d, int(causal), float(scale), _stream(stream))
    _check("fa_forward_fp32_out", code)
    return o, lse


def forward_f32(q, k, v, causal: bool, scale: float, o=None, lse=None, stream=None):
    """fp32 forward via fa_forward_f32."""
    return _forward("fa_forward_f32", torch.float32, q, k, v, causal, scale, o, lse, stream)


def _layout(block_mask, N, device):
    nb = (N + 63) // 64
    _require(block_mask, "block_mask", torch.uint8, (nb, nb))
    if block_mask.device != device:
        raise ValueError("block_mask must be on the same device as q")
    return block_mask


def _forward(fn, dtype, q, k, v, causal, scale, o, lse, stream, window=None, layout=None):
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k)
    _require(q, "q", dtype, (B, Hq, N, d))
    _require(k, "k", dtype, (B, Hkv, N, d))
    _require(v, "v", dtype, (B, Hkv, N, d))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require(o, "o", dtype, (B, Hq, N, d))
    _require(lse, "lse", torch.float32, (B, Hq, N))
    extra = () if window is None else (int(window),)
    lay = () if layout is None else (layout.data_ptr(),)
    code = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), *lay,
                            B, Hq, Hkv, N, d, int(causal), *extra, float(scale), _stream(stream))
    _check(fn, code)
    return o, lse


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))


def decode_forward(q, k, v, causal: bool, scale: float, o=None, lse=None, workspace=None, stream=None,
                   step: str = "all"):
    """bf16 forward of Nq new queries against an Nk-token key/value cache via
    fa_decode_forward (step "all"), or only its split or merge kernel (fa_decode_split /
    fa_decode_merge).  q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d].  Returns (o, lse)."""
    fn = {"all": "fa_decode_forward", "split": "fa_decode_split", "merge": "fa_decode_merge"}[step]
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _require(q, "q", torch.bfloat16, (B, Hq, Nq, d))
    _require(k, "k", torch.bfloat16, (B, Hkv, Nk, d))
    _require(v, "v", torch.bfloat16, (B, Hkv, Nk, d))
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o, "o", torch.bfloat16, (B, Hq, Nq, d))
    _require(lse, "lse", torch.float32, (B, Hq, Nq))
    if workspace is None:
        nbytes = decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    code = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale), _stream(stream))
    _check(fn, code)
    return o, lse


def decode_paged_forward(q, k_pages, v_pages, block_table, seq_lens, max_seq_len: int, causal: bool, scale: float,
                         o=None, lse=None, workspace=None, stream=None, step: str = "all"):
    """bf16 decode against a paged cache via fa_decode_paged_forward (or its split /
    merge kernel alone).  q [B,Hq,Nq,d]; k_pages, v_pages [num_pages,Hkv,page_size,d];
    block_table int32 [B,max_blocks]; seq_lens int32 [B].  Returns (o, lse)."""
    fn = {"all": "fa_decode_paged_forward", "split": "fa_decode_paged_split", "merge": "fa_decode_paged_merge"}[step]
    lib = load_library()
    if q.dim() != 4 or k_pages.dim() != 4:
        raise ValueError("q must be [B, Hq, Nq, d] and the pools [num_pages, Hkv, page_size, d]")
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page_size = k_pages.shape[:3]
    max_blocks = block_table.shape[1]
    _require(q, "q", torch.bfloat16, (B, Hq, Nq, d))
    _require(k_pages, "k_pages", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _require(v_pages, "v_pages", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _require(block_table, "block_table", torch.int32, (B, max_blocks))
    _require(seq_lens, "seq_lens", torch.int32, (B,))
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o, "o", torch.bfloat16, (B, Hq, Nq, d))
    _require(lse, "lse", torch.float32, (B, Hq, Nq))
    if workspace is None:
        nbytes = decode_workspace_bytes(B, Hq, Hkv, Nq, max_seq_len, d)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    code = getattr(lib, fn)(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                            seq_lens.data_ptr(), o.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), B, Hq, Hkv, Nq, int(max_seq_len),
                            num_pages, page_size, max_blocks, d, int(causal), float(scale), _stream(stream))
    _check(fn, code)
    return o, lse


def workspace_bytes(B: int, Hq: int, N: int) -> int:
    return int(load_library().fa_backward_workspace_bytes(B, Hq, N))


def fused_workspace_bytes(B: int, Hq: int, N: int, d: int) -> int:
    return int(load_library().fa_backward_fused_workspace_bytes(B, Hq, N, d))


def backward(q, k, v, o, do, lse, causal: bool, scale: float, dq=None, dk=None, dv=None,
             workspace=None, stream=None, window=None, block_mask=None, fused: bool = False):
    """bf16 backward via fa_backward (or fa_backward_window when ``window`` is given,
    fa_backward_blocksparse with ``block_mask``, or the fused alternative
    fa_backward_fused with ``fused=True``).  Returns (dq, dk, dv)."""
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k)
    for t, name, shp in ((q, "q", (B, Hq, N, d)), (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d)),
                         (o, "o", (B, Hq, N, d)), (do, "do", (B, Hq, N, d))):
        _require(t, name, torch.bfloat16, shp)
    _require(lse, "lse", torch.float32, (B, Hq, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", torch.bfloat16, (B, Hq, N, d))
    _require(dk, "dk", torch.bfloat16, (B, Hkv, N, d))
    _require(dv, "dv", torch.bfloat16, (B, Hkv, N, d))
    if fused and (window is not None or block_mask is not None):
        raise ValueError("the fused backward has no window or block-sparse form")
    nbytes = fused_workspace_bytes(B, Hq, N, d) if fused else workspace_bytes(B, Hq, N)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fn = "fa_backward_fused" if fused else ("fa_backward" if window is None else "fa_backward_window")
    extra = () if window is None else (int(window),)
    lay = ()
    if block_mask is not None:
        fn = "fa_backward_blocksparse"
        lay = (_layout(block_mask, N, q.device).data_ptr(),)
    code = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *lay,
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            B, Hq, Hkv, N, d, int(causal), *extra, float(scale), _stream(stream))
    _check(fn, code)
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, causal: bool, scale: float, dq=None, dk=None, dv=None, stream=None):
    """bf16 backward via fa_backward_noalloc (no workspace: the library's static scratch,
    at most 2^21 query rows).  Returns (dq, dk, dv)."""
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k)
    for t, name, shp in ((q, "q", (B, Hq, N, d)), (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d)),
                         (o, "o", (B, Hq, N, d)), (do, "do", (B, Hq, N, d))):
        _require(t, name, torch.bfloat16, shp)
    _require(lse, "lse", torch.float32, (B, Hq, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, "dq", torch.bfloat16, (B, Hq, N, d))
    _require(dk, "dk", torch.bfloat16, (B, Hkv, N, d))
    _require(dv, "dv", torch.bfloat16, (B, Hkv, N, d))
    code = lib.fa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   B, Hq, Hkv, N, d, int(causal), float(scale), _stream(stream))
    _check("fa_backward_noalloc", code)
    return dq, dk, dv


def backward_steps(q, k, v, o, do, lse, causal: bool, scale: float, dq, dk, dv, workspace,
                   stream=None, steps=("pre", "dkdv", "dq"), window=None, block_mask=None):
    """Enqueue the named backward steps in order: "pre" (fa_backward_preprocess), then
    "dkdv" and "dq" (fa_backward_dkdv / _dq, or their _window and _blocksparse forms);
    "pre_dq" (fa_backward_preprocess_dq and its forms: the preprocess and dQ in one
    kernel), then "dkdv", as fa_backward runs them; or the fused alternative's "fused"
    and "convert" (fa_backward_dkdv_dq, fa_backward_dq_convert; the workspace then needs
    fused_workspace_bytes, and "pre" also zeroes its accumulator).

    Preallocated outputs and workspace are required; this is the form the benchmark
    uses to time each kernel on its own.
    """
    lib = load_library()
    B, Hq, Hkv, N, d = _shape(q, k)
    st = _stream(stream)
    wsb = workspace.numel() * workspace.element_size()
    for step in steps:
        if step == "pre":
            code = lib.fa_backward_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                              wsb, B, Hq, N, d, st)
        elif step == "fused":
            if window is not None or block_mask is not None:
                raise ValueError("the fused backward has no window or block-sparse form")
            code = lib.fa_backward_dkdv_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                           workspace.data_ptr(), wsb, dk.data_ptr(), dv.data_ptr(),
                                           B, Hq, Hkv, N, d, int(causal), float(scale), st)
        elif step == "convert":
            code = lib.fa_backward_dq_convert(workspace.data_ptr(), wsb, dq.data_ptr(), B, Hq, N, d, float(scale), st)
        elif step == "dkdv" and block_mask is not None:
            code = lib.fa_backward_dkdv_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                                    workspace.data_ptr(), wsb, dk.data_ptr(), dv.data_ptr(),
                                                    _layout(block_mask, N, q.device).data_ptr(),
                                                    B, Hq, Hkv, N, d, int(causal), float(scale), st)
        elif step == "dq" and block_mask is not None:
            code = lib.fa_backward_dq_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                                  workspace.data_ptr(), wsb, dq.data_ptr(),
                                                  _layout(block_mask, N, q.device).data_ptr(),
                                                  B, Hq, Hkv, N, d, int(causal), float(scale), st)
        elif step == "dkdv":
            fn = "fa_backward_dkdv" if window is None else "fa_backward_dkdv_window"
            extra = () if window is None else (int(window),)
            code = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                    workspace.data_ptr(), wsb, dk.data_ptr(), dv.data_ptr(),
                                    B, Hq, Hkv, N, d, int(causal), *extra, float(scale), st)
        elif step == "pre_dq" and block_mask is not None:
            code = lib.fa_backward_preprocess_dq_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                             do.data_ptr(), lse.data_ptr(), workspace.data_ptr(), wsb,
                                                             dq.data_ptr(), _layout(block_mask, N, q.device).data_ptr(),
                                                             B, Hq, Hkv, N, d, int(causal), float(scale), st)
        elif step == "pre_dq":
            fn = "fa_backward_preprocess_dq" if window is None else "fa_backward_preprocess_dq_window"
            extra = () if window is None else (int(window),)
            code = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), workspace.data_ptr(), wsb, dq.data_ptr(),
                                    B, Hq, Hkv, N, d, int(causal), *extra, float(scale), st)
        elif step == "dq":
            fn = "fa_backward_dq" if window is None else "fa_backward_dq_window"
            extra = () if window is None else (int(window),)
            code = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                    workspace.data_ptr(), wsb, dq.data_ptr(),
                                    B, Hq, Hkv, N, d, int(causal), *extra, float(scale), st)
        else:
            raise ValueError(step)
        _check({"pre": "fa_backward_preprocess", "pre_dq": "fa_backward_preprocess_dq",
                "fused": "fa_backward_dkdv_dq"}.get(step, f"fa_backward_{step}"), code)
