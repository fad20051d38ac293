"""MI355X-native chunked gated delta rule: forward pass, decode, backward pass.

The compute lives in ``libgdn.so`` (hand-written HIP for gfx950 behind the C
ABI of ``include/gdn.h``); ``binding`` mirrors that ABI with ctypes and
``ops`` wraps it for torch tensors.  Importing this package does not load the
library; the first call does, and raises if it has not been built.
"""
from .ops import (backward, chunk_gated_delta_rule, causal_conv1d, chunk_prepare, decode_step, forward, forward_fused, forward_packed, forward_segmented,
                  gated_rmsnorm, num_pieces,
                  piece_compose, plan_pieces, problem_for, scan_carry, scan_emit, scan_head_carry,
                  scan_tail_emit, segment_bounds, segment_compose, split_wy)

__all__ = ["backward", "chunk_gated_delta_rule", "causal_conv1d", "gated_rmsnorm", "chunk_prepare", "decode_step", "forward", "forward_fused", "forward_packed", "forward_segmented", "num_pieces",
           "piece_compose", "plan_pieces", "problem_for", "scan_carry", "scan_emit", "scan_head_carry",
           "scan_tail_emit", "segment_bounds", "segment_compose", "split_wy"]
__version__ = "0.1.0"
