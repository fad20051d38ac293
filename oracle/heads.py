"""Grouped key heads (test infrastructure, like the rest of ``oracle/``).

"RFC(qwen35): TP Phase 2", section "Partition Contract", gives the linear
attention separate key and value head counts: q and k have H_qk heads, v, the
gates and the recurrent state [H_v, K, V] have H_v heads.  The Ulysses
context-parallelism page names the pairing: each key head is repeated in
grouped order, [kv0, kv0, kv1, kv1] rather than tiled [kv0, kv1, kv0, kv1], so
value head h reads key head h // (H_v / H_qk).

The definition is therefore the ungrouped recurrence on q and k with each key
head repeated H_v / H_qk times in place.
"""
import numpy as np


def expand_key_heads(x, H_v, axis=-2):
    """q or k with H_qk heads on `axis` (the head axis: [..., H_qk, K] by
    default) repeated in grouped order to H_v heads."""
    x = np.asarray(x)
    H_qk = x.shape[axis]
    if H_qk < 1 or H_v % H_qk != 0:
        raise ValueError(f"value heads {H_v} are not a multiple of key heads {H_qk}")
    return np.repeat(x, H_v // H_qk, axis=axis)
