"""CPU float64 oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the package's smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .attention import (attention_backward, attention_forward, decode_forward,
                        head_backward, head_forward, head_probs, paged_decode_forward, paged_gather)
from .online import head_forward_merged, merge_states, online_softmax_states, tile_state

__all__ = ["attention_forward", "attention_backward", "decode_forward", "paged_decode_forward", "paged_gather",
           "head_forward", "head_backward",
           "head_probs", "head_forward_merged", "merge_states", "tile_state", "online_softmax_states"]
