"""MI355X-native chunked gated delta rule forward pass.

The compute lives in ``libgdn.so`` (hand-written HIP for gfx950 behind the C
ABI of ``include/gdn.h``); ``binding`` mirrors that ABI with ctypes and
``ops`` wraps it for torch tensors.  Importing this package does not load the
library; the first call does, and raises if it has not been built.
"""
from .ops import (chunk_prepare, decode_step, forward, forward_segmented, problem_for, scan_carry,
                  scan_emit, scan_head_carry, segment_bounds, segment_compose, split_wy)

__all__ = ["chunk_prepare", "decode_step", "forward", "forward_segmented", "problem_for",
           "scan_carry", "scan_emit", "scan_head_carry", "segment_bounds", "segment_compose", "split_wy"]
__version__ = "0.1.0"
