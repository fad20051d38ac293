"""fp64 reverse mode of the gated delta rule (test infrastructure).

The MaxText PR "Add context parallelism to the Gated Delta Net" checks its
backward pass against the single-device recurrence (section "Tests") but
prints no backward algorithm.  The definition used here is therefore the
chain rule applied to the token recurrence of ``recurrence.py``: the
vector-Jacobian product of the map (q, k, v, g, beta, h0) -> (o, hT) for a
given (dl/do, dl/dhT), taken token by token from the last token back.  The
arithmetic lives in ``gdn_oracle.c`` (``backward_chain``); this module only
marshals arrays.  It keeps every state of a chain in memory, so it is meant
for test sizes.
"""
import ctypes

import numpy as np

from .recurrence import load_library, _f64, _ptr, _dp, _ip

_READY = False


def _lib():
    global _READY
    lib = load_library()
    if not _READY:
        lib.gdn_oracle_backward.restype = ctypes.c_int
        lib.gdn_oracle_backward.argtypes = [ctypes.c_int] * 5 + [_dp] * 14 + [ctypes.c_int]
        lib.gdn_oracle_backward_packed.restype = ctypes.c_int
        lib.gdn_oracle_backward_packed.argtypes = ([ctypes.c_int, _ip] + [ctypes.c_int] * 3
                                                   + [_dp] * 14 + [ctypes.c_int])
        _READY = True
    return lib


def backward(q, k, v, g, beta, h0, do, dhT=None, nthreads=0):
    """Batch mode.  Shapes as ``recurrence.forward``; do [B,S,H,V]; dhT [B,H,K,V] or None.

    Returns (dq, dk, dv, dg, dbeta, dh0) in float64, each in the layout of its
    input (dh0 is returned whether or not h0 was given: the gradient at h0 = 0).
    """
    q, k, v, g, beta, h0, do, dhT = (_f64(a) for a in (q, k, v, g, beta, h0, do, dhT))
    B, S, H, K = k.shape
    V = v.shape[-1]
    assert q.shape == k.shape and v.shape == (B, S, H, V) and do.shape == v.shape
    assert g.shape == (B, S, H) and beta.shape == (B, S, H)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    dh0 = np.zeros((B, H, K, V))
    rc = _lib().gdn_oracle_backward(B, S, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(h0), _ptr(do), _ptr(dhT), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                    int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle backward failed")
    return dq, dk, dv, dg, dbeta, dh0


def backward_packed(cu_seqlens, q, k, v, g, beta, h0, do, dhT=None, nthreads=0):
    """Packed mode.  Shapes as ``recurrence.forward_packed``; do [T,H,V]; dhT [N,H,K,V]."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    q, k, v, g, beta, h0, do, dhT = (_f64(a) for a in (q, k, v, g, beta, h0, do, dhT))
    T, H, K = k.shape
    V = v.shape[-1]
    N = len(cu) - 1
    assert cu[-1] == T and do.shape == v.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    dh0 = np.zeros((N, H, K, V))
    rc = _lib().gdn_oracle_backward_packed(
        N, cu.ctypes.data_as(_ip), H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(h0), _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
        _ptr(dh0), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle packed backward failed")
    return dq, dk, dv, dg, dbeta, dh0
