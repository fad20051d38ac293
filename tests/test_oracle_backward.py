"""Pins of the fp64 reverse-mode oracle against things other than itself (CPU only).

* central finite differences of the forward oracle (the definition of a
  derivative, with an O(eps^2) error bound), for every input, in batch and
  packed mode, with nonzero h0 and dl/dhT;
* the scalar one-token case (K = V = 1) differentiated by hand;
* the beta = 0 closed form, where k and v drop out of the recurrence;
* the chunked algebra of a backward pass (``oracle.chunked_backward``), an
  independent second derivation, at several chunk sizes and ragged tails.
"""
import numpy as np
import pytest

import oracle
from oracle.backward import backward, backward_packed
from oracle.chunked import chunked_backward


def _problem(rng, B, S, H, K, V, h0=True):
    q = rng.standard_normal((B, S, H, K))
    k = rng.standard_normal((B, S, H, K)) * 0.5
    v = rng.standard_normal((B, S, H, V))
    g = -np.abs(rng.standard_normal((B, S, H))) * 0.3
    beta = rng.uniform(0.0, 1.0, (B, S, H))
    s0 = rng.standard_normal((B, H, K, V)) if h0 else None
    do = rng.standard_normal((B, S, H, V))
    dhT = rng.standard_normal((B, H, K, V))
    return q, k, v, g, beta, s0, do, dhT


def _directional(loss, xs, n, d, eps=1e-5):
    a = list(xs)
    a[n] = xs[n] + eps * d
    lp = loss(*a)
    a[n] = xs[n] - eps * d
    lm = loss(*a)
    return (lp - lm) / (2 * eps)


@pytest.mark.parametrize("shape", [(1, 7, 2, 3, 4), (2, 5, 1, 4, 2), (1, 1, 1, 2, 3)])
def test_backward_matches_finite_differences(shape):
    rng = np.random.default_rng(11)
    q, k, v, g, beta, h0, do, dhT = _problem(rng, *shape)
    grads = backward(q, k, v, g, beta, h0, do, dhT)

    def loss(q, k, v, g, beta, h0):
        o, hT = oracle.forward(q, k, v, g, beta, h0)
        return float((o * do).sum() + (hT * dhT).sum())

    xs = [q, k, v, g, beta, h0]
    for n, grad in enumerate(grads):
        for _ in range(2):
            d = rng.standard_normal(xs[n].shape)
            fd = _directional(loss, xs, n, d)
            an = float((grad * d).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (n, fd, an)


def test_packed_backward_matches_finite_differences():
    rng = np.random.default_rng(12)
    cu = np.array([0, 3, 3, 8, 9], dtype=np.int32)
    T, H, K, V = 9, 2, 3, 2
    q, k, v, g, beta, _, do, _ = (x[0] if x is not None else None
                                  for x in _problem(rng, 1, T, H, K, V, h0=False))
    h0 = rng.standard_normal((4, H, K, V))
    dhT = rng.standard_normal((4, H, K, V))
    grads = backward_packed(cu, q, k, v, g, beta, h0, do, dhT)

    def loss(q, k, v, g, beta, h0):
        o, hT = oracle.forward_packed(cu, q, k, v, g, beta, h0)
        return float((o * do).sum() + (hT * dhT).sum())

    xs = [q, k, v, g, beta, h0]
    for n, grad in enumerate(grads):
        d = rng.standard_normal(xs[n].shape)
        fd = _directional(loss, xs, n, d)
        an = float((grad * d).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (n, fd, an)
    # the empty sequence passes dl/dhT straight through to dl/dh0
    np.testing.assert_array_equal(grads[5][1], dhT[1])


def test_scalar_token_by_hand():
    # K = V = 1, one token: h1 = a (1 - b k^2) h0 + b k v, o = h1 q,
    # loss = do * o + dhT * h1, a = exp(g).
    q, k, v, g, b, h0, do, dhT = 0.7, -1.3, 0.4, -0.25, 0.6, 1.1, -0.9, 0.35
    a = np.exp(g)
    h1 = a * (1 - b * k * k) * h0 + b * k * v
    dh1 = q * do + dhT
    want = dict(dq=h1 * do, dk=dh1 * (-2 * a * b * k * h0 + b * v), dv=dh1 * b * k,
                dg=dh1 * a * (1 - b * k * k) * h0, dbeta=dh1 * (-a * k * k * h0 + k * v),
                dh0=dh1 * a * (1 - b * k * k))
    arr = lambda x: np.full((1, 1, 1, 1), x)
    got = backward(arr(q), arr(k), arr(v), np.full((1, 1, 1), g), np.full((1, 1, 1), b),
                   arr(h0), arr(do), arr(dhT))
    for name, x in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], got):
        assert np.allclose(x.ravel(), want[name], rtol=1e-14, atol=0), name


def test_beta_zero_closed_form():
    # beta = 0: h_t = exp(G_t) h0, o_t = exp(G_t) h0^T q_t; k and v drop out.
    rng = np.random.default_rng(13)
    q, k, v, g, _, h0, do, dhT = _problem(rng, 1, 9, 2, 4, 3)
    beta = np.zeros(g.shape)
    dq, dk, dv, dg, dbeta, dh0 = backward(q, k, v, g, beta, h0, do, dhT)
    assert not dk.any() and not dv.any()
    G = np.cumsum(g, axis=1)                                     # [1,S,H]
    e = np.exp(G)
    want_dq = e[..., None] * np.einsum("hkv,shv->shk", h0[0], do[0])[None]
    assert np.allclose(dq, want_dq, rtol=1e-13, atol=1e-15)
    want_dh0 = (np.einsum("sh,shk,shv->hkv", e[0], q[0], do[0])
                + np.exp(G[0, -1])[:, None, None] * dhT[0])
    assert np.allclose(dh0[0], want_dh0, rtol=1e-13, atol=1e-15)
    # dl/dG_t = e_t (q_t^T h0 do_t) + [t = S-1] exp(G_S) <h0, dhT>; dg is its reverse cumsum
    dG = e[0] * np.einsum("shk,hkv,shv->sh", q[0], h0[0], do[0])
    dG[-1] += np.exp(G[0, -1]) * np.einsum("hkv,hkv->h", h0[0], dhT[0])
    want_dg = np.cumsum(dG[::-1], axis=0)[::-1]
    assert np.allclose(dg[0], want_dg, rtol=1e-12, atol=1e-15)
    # d/dbeta at beta = 0: delta = beta (v - h^T k) with h = exp(G_t) h0 (pre-write state)
    S = q.shape[1]
    for t in range(S):
        for hh in range(2):
            hprev = np.exp(G[0, t, hh]) * h0[0, hh]
            e_t = v[0, t, hh] - hprev.T @ k[0, t, hh]
            # the write k e^T reaches o_s (s >= t) and hT through later decays only
            dht = np.exp(G[0, -1, hh] - G[0, t, hh]) * dhT[0, hh]
            for s in range(t, S):
                dht = dht + np.exp(G[0, s, hh] - G[0, t, hh]) * np.outer(q[0, s, hh], do[0, s, hh])
            assert np.isclose(dbeta[0, t, hh], k[0, t, hh] @ dht @ e_t, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("S,C", [(37, 8), (64, 16), (50, 50), (9, 1), (40, 64)])
def test_chunked_backward_matches_recurrence(S, C):
    rng = np.random.default_rng(14)
    q, k, v, g, beta, h0, do, dhT = _problem(rng, 2, S, 2, 5, 6)
    ref = backward(q, k, v, g, beta, h0, do, dhT)
    got = chunked_backward(q, k, v, g, beta, C, h0, do, dhT)
    for r, x in zip(ref, got):
        assert np.abs(x - r).max() <= 1e-12 * np.abs(r).max()


def test_packed_backward_equals_per_sequence_batch():
    rng = np.random.default_rng(15)
    cu = np.array([0, 5, 12, 20], dtype=np.int32)
    q, k, v, g, beta, _, do, _ = (x[0] if x is not None else None
                                  for x in _problem(rng, 1, 20, 2, 3, 4, h0=False))
    h0 = rng.standard_normal((3, 2, 3, 4))
    dhT = rng.standard_normal((3, 2, 3, 4))
    got = backward_packed(cu, q, k, v, g, beta, h0, do, dhT)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        ref = backward(q[None, a:b], k[None, a:b], v[None, a:b], g[None, a:b], beta[None, a:b],
                       h0[n:n + 1], do[None, a:b], dhT[n:n + 1])
        for r, x in zip(ref[:5], got[:5]):
            np.testing.assert_array_equal(x[a:b], r[0])
        np.testing.assert_array_equal(got[5][n], ref[5][0])
