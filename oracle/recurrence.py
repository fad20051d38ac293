"""fp64 token recurrence of the gated delta rule (test infrastructure).

The definition the whole path must reproduce.  The chunked equations of the
MaxText PR "Add context parallelism to the Gated Delta Net" (section "Why")
are a rearrangement of it; the page names it the "sequential recurrence"
(section "Limitation") and tests against the "single-device recurrence"
(section "Tests").  Per token, with the K-major state h (K x V):

    h <- exp(g_t) h ;  delta = beta_t (v_t - h^T k_t) ;  h <- h + k_t delta^T ;
    o_t = h^T q_t

The arithmetic lives in ``gdn_oracle.c``; this module only marshals arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def load_library():
    """Load ``liboracle.so``, compiling it with gcc first if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.gdn_oracle_forward.restype = ctypes.c_int
        lib.gdn_oracle_forward.argtypes = [ctypes.c_int] * 5 + [_dp] * 8 + [ctypes.c_int]
        lib.gdn_oracle_forward_packed.restype = ctypes.c_int
        lib.gdn_oracle_forward_packed.argtypes = ([ctypes.c_int, _ip] + [ctypes.c_int] * 3
                                                  + [_dp] * 8 + [ctypes.c_int])
        _LIB = lib
    return _LIB


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def forward(q, k, v, g, beta, h0=None, nthreads=0, want_o=True):
    """Batch mode.  q,k [B,S,H,K]; v [B,S,H,V]; g,beta [B,S,H]; h0 [B,H,K,V] or None.

    Returns (o [B,S,H,V] or None, hT [B,H,K,V]) in float64.  ``q`` may be None
    when ``want_o`` is False (a pass that only carries the state).
    """
    k, v, g, beta = _f64(k), _f64(v), _f64(g), _f64(beta)
    q = _f64(q) if want_o else None
    B, S, H, K = k.shape
    V = v.shape[-1]
    assert v.shape == (B, S, H, V) and g.shape == (B, S, H) and beta.shape == (B, S, H)
    if q is not None:
        assert q.shape == (B, S, H, K)
    h0 = _f64(h0)
    if h0 is not None:
        assert h0.shape == (B, H, K, V)
    o = np.zeros((B, S, H, V)) if want_o else None
    hT = np.zeros((B, H, K, V))
    rc = load_library().gdn_oracle_forward(B, S, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle forward failed")
    return o, hT


def forward_packed(cu_seqlens, q, k, v, g, beta, h0=None, nthreads=0):
    """Packed mode.  q,k [T,H,K]; v [T,H,V]; g,beta [T,H]; h0 [N,H,K,V] or None.

    Sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1, T = cu_seqlens[N].
    Returns (o [T,H,V], hT [N,H,K,V]) in float64.
    """
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    q, k, v, g, beta, h0 = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(h0)
    T, H, K = k.shape
    V = v.shape[-1]
    N = len(cu) - 1
    assert cu[-1] == T
    o = np.zeros((T, H, V))
    hT = np.zeros((N, H, K, V))
    rc = load_library().gdn_oracle_forward_packed(
        N, cu.ctypes.data_as(_ip), H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(h0), _ptr(o), _ptr(hT), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle packed forward failed")
    return o, hT


def decode_step(q, k, v, g, beta, state, nthreads=0):
    """One recurrent step for a batch of independent sequences.

    q,k [B,H,K]; v [B,H,V]; g,beta [B,H]; state [B,H,K,V].  Returns
    (o [B,H,V], new_state [B,H,K,V]): the recurrence over a single token.
    """
    o, hT = forward(np.asarray(q)[:, None], np.asarray(k)[:, None], np.asarray(v)[:, None],
                    np.asarray(g)[:, None], np.asarray(beta)[:, None], h0=state,
                    nthreads=nthreads)
    return o[:, 0], hT


def transition_pair(k, v, g, beta, nthreads=0):
    """(M, U) of the state map a token range induces: h_out = M h_in + U.

    The page's affine form (MaxText PR "Add context parallelism to the Gated
    Delta Net", section "Why": M_r is (B,H,K,K), U_r is (B,H,K,V)), taken by
    definition from the recurrence: U is the final state of a pass from the
    zero state, and M is the final state of a pass with every v_t = 0 started
    from the K x K identity (the map is linear in h_in when v = 0).

    k [B,S,H,K]; v [B,S,H,V]; g,beta [B,S,H].  Returns M [B,H,K,K], U [B,H,K,V].
    """
    k = _f64(k)
    B, S, H, K = k.shape
    eye = np.broadcast_to(np.eye(K), (B, H, K, K))
    _, M = forward(None, k, np.zeros((B, S, H, K)), g, beta, h0=eye, nthreads=nthreads,
                   want_o=False)
    _, U = forward(None, k, v, g, beta, h0=None, nthreads=nthreads, want_o=False)
    return M, U
