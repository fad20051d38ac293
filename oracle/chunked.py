"""Chunked (WY) form of the gated delta rule in NumPy fp64 (test infrastructure).

Follows the affine chunk equations of the MaxText PR "Add context parallelism
to the Gated Delta Net (Qwen3-Next / Qwen3.5)", section "Why":

    h_out = (gamma I - k_tilde^T w) h + k_tilde^T u  ==  M h + U
    o     = (q_g - attn_i w) h + attn_i u

and the low-rank composition of M from the same page, section
"Implementation":  M_new = gamma M - k_tilde^T (w M).

The page leaves gamma, k_tilde, w, u, q_g and attn_i undefined.  The reading
taken here (the unique one that makes the equations reproduce the token
recurrence in ``recurrence.py`` at every chunk size, which the tests check
against it) is, for a chunk of L
tokens with local indices r, s and within-chunk cumulative log-decay
G_r = g_1 + ... + g_r:

    A[r,s]    = beta_r exp(G_r - G_s) k_r . k_s    (s < r; zero elsewhere)
    T         = (I + A)^{-1}                       (unit lower triangular)
    w         = T diag(beta_r exp(G_r)) K           u = T diag(beta_r) V
    k_tilde_s = exp(G_L - G_s) k_s                  gamma = exp(G_L)
    q_g[r]    = exp(G_r) q_r
    attn[r,s] = exp(G_r - G_s) q_r . k_s           (s <= r, diagonal included)

Decay ratios are formed as exp(G_r - G_s) with s <= r, never as a quotient of
two exponentials.  A tail chunk simply has L < C tokens.
"""
import numpy as np
from scipy.linalg import solve_triangular


def _chunk_terms(q, k, v, g, beta):
    """All chunk-local quantities for one chain's chunk (2-D arrays [L, .])."""
    L = k.shape[0]
    G = np.cumsum(g)
    diff = G[:, None] - G[None, :]                   # G_r - G_s
    lower = np.tril(np.ones((L, L), dtype=bool), -1)  # s < r
    causal = np.tril(np.ones((L, L), dtype=bool), 0)  # s <= r
    decay = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    A = np.where(lower, beta[:, None] * decay * (k @ k.T), 0.0)
    I_A = np.eye(L) + A
    w = solve_triangular(I_A, (beta * np.exp(G))[:, None] * k, lower=True, unit_diagonal=True)
    u = solve_triangular(I_A, beta[:, None] * v, lower=True, unit_diagonal=True)
    gamma = np.exp(G[-1]) if L else 1.0
    k_tilde = np.exp(G[-1] - G)[:, None] * k if L else k
    terms = dict(G=G, A=A, w=w, u=u, gamma=gamma, k_tilde=k_tilde)
    if q is not None:
        terms["q_g"] = np.exp(G)[:, None] * q
        terms["attn"] = np.where(causal, decay * (q @ k.T), 0.0)
    return terms


def _chunks(S, C):
    return [(c0, min(c0 + C, S)) for c0 in range(0, S, C)]


def chunk_wy(k, v, g, beta, C):
    """WY factors of every chunk, batch layout.

    k [B,S,H,K], v [B,S,H,V], g,beta [B,S,H] -> w [B,Nc,H,C,K], u [B,Nc,H,C,V]
    with Nc = ceil(S/C).  Rows past the end of a tail chunk are zero (they are
    the padded positions, whose beta is zero).
    """
    k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (k, v, g, beta))
    B, S, H, K = k.shape
    V = v.shape[-1]
    spans = _chunks(S, C)
    w = np.zeros((B, len(spans), H, C, K))
    u = np.zeros((B, len(spans), H, C, V))
    for b in range(B):
        for h in range(H):
            for j, (c0, c1) in enumerate(spans):
                t = _chunk_terms(None, k[b, c0:c1, h], v[b, c0:c1, h], g[b, c0:c1, h],
                                 beta[b, c0:c1, h])
                w[b, j, h, :c1 - c0] = t["w"]
                u[b, j, h, :c1 - c0] = t["u"]
    return w, u


def chunk_transition(k, v, g, beta):
    """(M_c, U_c) of one chunk of one chain: M_c = gamma I - k_tilde^T w, U_c = k_tilde^T u."""
    t = _chunk_terms(None, *(np.asarray(a, dtype=np.float64) for a in (k, v, g, beta)))
    K = t["k_tilde"].shape[1]
    return t["gamma"] * np.eye(K) - t["k_tilde"].T @ t["w"], t["k_tilde"].T @ t["u"]


def chunked_forward(q, k, v, g, beta, C, h0=None):
    """Chunk-by-chunk forward, batch layout; returns (o [B,S,H,V], hT [B,H,K,V])."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, S, H, K = k.shape
    V = v.shape[-1]
    o = np.zeros((B, S, H, V))
    hT = np.zeros((B, H, K, V))
    for b in range(B):
        for hh in range(H):
            h = np.zeros((K, V)) if h0 is None else np.array(h0[b, hh], dtype=np.float64)
            for c0, c1 in _chunks(S, C):
                t = _chunk_terms(q[b, c0:c1, hh], k[b, c0:c1, hh], v[b, c0:c1, hh],
                                 g[b, c0:c1, hh], beta[b, c0:c1, hh])
                delta = t["u"] - t["w"] @ h                       # the chunk's delta rows
                o[b, c0:c1, hh] = t["q_g"] @ h + t["attn"] @ delta  # eq. for o
                h = t["gamma"] * h + t["k_tilde"].T @ delta        # eq. for h_out
            hT[b, hh] = h
    return o, hT


def lowrank_segment_pair(k, v, g, beta, C):
    """(M_r, U_r) of a whole token range by chunk-wise low-rank composition.

    Phase 1 of the three-phase pass (MaxText PR, section "Implementation"):
    a zero-state pass that carries M alongside the state, with
    M <- gamma M - k_tilde^T (w M) starting from M = I, and
    U <- gamma U + k_tilde^T (u - w U) starting from U = 0.
    k [B,S,H,K] ... -> M [B,H,K,K], U [B,H,K,V].
    """
    k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (k, v, g, beta))
    B, S, H, K = k.shape
    V = v.shape[-1]
    M = np.zeros((B, H, K, K))
    U = np.zeros((B, H, K, V))
    for b in range(B):
        for hh in range(H):
            m, uu = np.eye(K), np.zeros((K, V))
            for c0, c1 in _chunks(S, C):
                t = _chunk_terms(None, k[b, c0:c1, hh], v[b, c0:c1, hh], g[b, c0:c1, hh],
                                 beta[b, c0:c1, hh])
                m = t["gamma"] * m - t["k_tilde"].T @ (t["w"] @ m)
                uu = t["gamma"] * uu + t["k_tilde"].T @ (t["u"] - t["w"] @ uu)
            M[b, hh], U[b, hh] = m, uu
    return M, U
