"""Exact IO-aware attention for MI355X (gfx950): hand-written HIP kernels behind a C ABI.

The compute path is ``libfa_mi355x.so`` (built from ``csrc/``); this package only
marshals torch tensors (device memory and streams) into its entry points.
Submodules ``inputs`` and ``measure`` are plain Python and need no GPU.
"""
__all__ = ["api", "inputs", "measure", "build"]
