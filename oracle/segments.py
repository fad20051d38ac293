"""Exclusive prefix scan over segment transition pairs (test infrastructure).

Phase 2 of the three-phase pass in the MaxText PR "Add context parallelism to
the Gated Delta Net" (section "Implementation"): every segment r collapses to
(M_r, U_r) with h_out = M_r h_in + U_r (section "Why"), and the state entering
segment r is the exclusive scan of those affine maps seeded with the initial
state:  h_in(0) = h0,  h_in(r+1) = M_r h_in(r) + U_r.  The inclusive end,
M_{R-1} h_in(R-1) + U_{R-1}, is the final state.
"""
import numpy as np


def exclusive_scan(M, U, h0=None):
    """M [R,B,H,K,K], U [R,B,H,K,V], h0 [B,H,K,V] or None.

    Returns (h_in [R,B,H,K,V], h_final [B,H,K,V]) in float64.
    """
    M = np.asarray(M, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    R = M.shape[0]
    h = np.zeros(U.shape[1:]) if h0 is None else np.array(h0, dtype=np.float64)
    h_in = np.zeros(U.shape)
    for r in range(R):
        h_in[r] = h
        h = M[r] @ h + U[r]
    return h_in, h
