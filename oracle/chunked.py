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
    terms = dict(G=G, A=A, w=w, u=u, gamma=gamma, k_tilde=k_tilde, decay=decay)
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


def chunked_backward(q, k, v, g, beta, C, h0, do, dhT=None):
    """Gradients of the chunked form, batch layout: (dq, dk, dv, dg, dbeta, dh0).

    The chain rule taken through the chunk equations above rather than through
    the token recurrence, so it checks the chunk algebra of a backward pass
    against ``backward.backward``.  A forward sweep keeps the state h_c at the
    start of every chunk; a reverse sweep carries dh (dl/dh at the chunk's end)
    and, per chunk, with D = Dec (the causal decay ratios exp(G_r - G_s)),
    Kb = diag(beta exp(G)) K and Vb = diag(beta) V (so w = T Kb, u = T Vb):

        delta  = u - w h_c
        ddelta = attn^T do + k_tilde dh           (o and h_out both read delta)
        dh_c   = gamma dh + q_g^T do - w^T ddelta
        dattn  = causal(do delta^T);  dq_g = do h_c^T;  dk_tilde = delta dh^T
        dw     = -ddelta h_c^T;       du = ddelta
        dT     = du Vb^T + dw Kb^T;   dVb = T^T du;  dKb = T^T dw
        dA     = -strict_lower(T^T dT T^T)        (T = (I + A)^{-1})

    then every chunk quantity hands its gradient to q, k, v, beta and the
    cumulative decay G; dg is the reverse cumulative sum of dG in the chunk.
    """
    q, k, v, g, beta, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, do))
    B, S, H, K = k.shape
    V = v.shape[-1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    dh0 = np.zeros((B, H, K, V))
    spans = _chunks(S, C)
    for b in range(B):
        for hh in range(H):
            h = np.zeros((K, V)) if h0 is None else np.array(h0[b, hh], dtype=np.float64)
            starts, terms = [], []
            for c0, c1 in spans:
                t = _chunk_terms(q[b, c0:c1, hh], k[b, c0:c1, hh], v[b, c0:c1, hh],
                                 g[b, c0:c1, hh], beta[b, c0:c1, hh])
                starts.append(h)
                terms.append(t)
                h = t["gamma"] * h + t["k_tilde"].T @ (t["u"] - t["w"] @ h)
            dh = np.zeros((K, V)) if dhT is None else np.array(dhT[b, hh], dtype=np.float64)
            for (c0, c1), hc, t in reversed(list(zip(spans, starts, terms))):
                qq, kk, vv = q[b, c0:c1, hh], k[b, c0:c1, hh], v[b, c0:c1, hh]
                bb, dd = beta[b, c0:c1, hh], do[b, c0:c1, hh]
                L = c1 - c0
                G, D, A = t["G"], t["decay"], t["A"]
                eG = np.exp(G)
                T = np.linalg.inv(np.eye(L) + A)
                Kb, Vb = (bb * eG)[:, None] * kk, bb[:, None] * vv
                delta = t["u"] - t["w"] @ hc
                ddelta = t["attn"].T @ dd + t["k_tilde"] @ dh
                dh_c = t["gamma"] * dh + t["q_g"].T @ dd - t["w"].T @ ddelta
                causal = np.tril(np.ones((L, L), dtype=bool), 0)
                dattn = np.where(causal, dd @ delta.T, 0.0)
                dq_g = dd @ hc.T
                dk_tilde = delta @ dh.T
                dw = -ddelta @ hc.T
                dT = ddelta @ Vb.T + dw @ Kb.T
                dVb, dKb = T.T @ ddelta, T.T @ dw
                dA = np.tril(-(T.T @ dT @ T.T), -1)
                dKK = dA * bb[:, None] * D                       # A = beta_r D (K K^T)
                P = dattn * D                                    # attn = D (Q K^T)
                dq_ = eG[:, None] * dq_g + P @ kk
                dk_ = (P.T @ qq + np.exp(G[-1] - G)[:, None] * dk_tilde
                       + (bb * eG)[:, None] * dKb + dKK @ kk + dKK.T @ kk)
                dv_ = bb[:, None] * dVb
                db_ = (dVb * vv).sum(1) + (dKb * eG[:, None] * kk).sum(1) + (dA * D * (kk @ kk.T)).sum(1)
                dG = (dq_g * t["q_g"]).sum(1)
                ea = dattn * t["attn"]
                dG += ea.sum(1) - ea.sum(0)
                ek = (dk_tilde * t["k_tilde"]).sum(1)
                dG -= ek
                dG += (dKb * Kb).sum(1)
                eA = dA * A
                dG += eA.sum(1) - eA.sum(0)
                dG[-1] += ek.sum() + t["gamma"] * (hc * dh).sum()
                dq[b, c0:c1, hh], dk[b, c0:c1, hh], dv[b, c0:c1, hh] = dq_, dk_, dv_
                dbeta[b, c0:c1, hh] = db_
                dg[b, c0:c1, hh] = np.cumsum(dG[::-1])[::-1]
                dh = dh_c
            dh0[b, hh] = dh
    return dq, dk, dv, dg, dbeta, dh0
