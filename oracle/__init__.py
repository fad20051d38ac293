"""CPU oracle of the gated delta rule forward pass -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or execute anything in this package.  The
HIP product path never touches it, and it shares no code, header, table or
helper with that path.

Contents (every function cites the passage of the pages it follows):

* ``recurrence``  -- the definition: the fp64 token-by-token recurrence in C
  (``gdn_oracle.c``), plus the transition pair (M, U) of a token range, defined
  as the linear and constant parts of the state map that recurrence induces.
* ``chunked``     -- the chunked WY rearrangement (eq. for h_out and o in the
  MaxText PR "Add context parallelism to the Gated Delta Net", section "Why")
  and the low-rank composition of M (same page, section "Implementation"),
  in NumPy fp64.  An independent second algorithm used to cross-check the
  recurrence, and the oracle for the WY factors w, u.
* ``segments``    -- the exclusive prefix scan over (M_r, U_r) (same page,
  section "Implementation", phase 2).
* ``layers``      -- the depthwise causal conv before the core and the gated
  RMSNorm after it (MaxText PR, section "Implementation"; "RFC(qwen35): TP
  Phase 2", sections "Partition Contract" and "Execution Contract"); readings in its
  header.
* ``backward``    -- reverse mode: the chain rule applied to the token
  recurrence (the vector-Jacobian product for given dl/do, dl/dhT), fp64 in
  C; ``chunked.chunked_backward`` is the same gradient taken through the
  chunk equations, an independent second derivation.
* ``heads``       -- grouped key heads ("RFC(qwen35): TP Phase 2", section
  "Partition Contract"; grouped order from the Ulysses page): the ungrouped
  definition on q, k with each key head repeated in place.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, hand-worked fixtures under
``tests/golden/`` and the independent chunked algorithm; the backward pass
also against central finite differences of the forward.  The only thing left
unpinned is the bf16 tolerance margin of the GPU comparison, which the pages
do not print.
"""
from .recurrence import (forward, forward_packed, decode_step, transition_pair,
                         load_library)
from .chunked import (chunk_wy, chunked_forward, chunk_transition,
                      lowrank_segment_pair, chunked_backward)
from .backward import backward, backward_packed
from .segments import exclusive_scan
from .heads import expand_key_heads
from .layers import silu, causal_conv1d, causal_conv1d_packed, gated_rmsnorm

__all__ = [
    "forward", "forward_packed", "decode_step", "transition_pair", "load_library",
    "chunk_wy", "chunked_forward", "chunk_transition", "lowrank_segment_pair",
    "chunked_backward", "backward", "backward_packed",
    "exclusive_scan", "expand_key_heads", "silu", "causal_conv1d", "causal_conv1d_packed", "gated_rmsnorm",
]
