"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a hand-worked fixture, a closed form, an
invariant of the gated delta rule, or the independent chunked (WY) algorithm,
chosen so that a dropped term, a wrong sign, a misplaced decay, a transposed
operand or a wrong stride fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import make_inputs, make_packed_inputs, make_decode_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _chain_arrays(d):
    """Golden fixture (one chain) -> batch-layout arrays with B = H = 1."""
    k = np.array(d["k"], dtype=np.float64)[None, :, None, :]
    q = np.array(d["q"], dtype=np.float64)[None, :, None, :]
    v = np.array(d["v"], dtype=np.float64)[None, :, None, :]
    g = np.array(d["g"], dtype=np.float64)[None, :, None]
    beta = np.array(d["beta"], dtype=np.float64)[None, :, None]
    h0 = np.array(d["h0"], dtype=np.float64)[None, None]
    return q, k, v, g, beta, h0


@pytest.mark.parametrize("name", ["delta_rule_two_tokens.json", "overwrite_table.json"])
def test_hand_worked_fixtures(name):
    d = _golden(name)
    q, k, v, g, beta, h0 = _chain_arrays(d)
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    np.testing.assert_allclose(o[0, :, 0], np.array(d["o"]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hT[0, 0], np.array(d["hT"]), rtol=1e-13, atol=1e-13)


def _rand(seed, B=2, S=9, H=3, K=5, V=4, decay="config", h0_std=0.5):
    x = make_inputs(seed, B, S, H, K, V, 4, "f32", h0_std, decay)
    f64 = lambda a: None if a is None else a.astype(np.float64)
    return f64(x.q), f64(x.k), f64(x.v), f64(x.g), f64(x.beta), f64(x.h0)


def test_beta_zero_closed_form():
    """beta = 0: no writes, pure decay.  h_T = exp(sum g) h0, o_t = exp(G_t) h0^T q_t."""
    q, k, v, g, beta, h0 = _rand(1)
    beta = np.zeros_like(beta)
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    G = np.cumsum(g.astype(np.float64), axis=1)                      # [B,S,H]
    exp_o = np.einsum("bshk,bhkv->bshv", q.astype(np.float64), h0.astype(np.float64))
    exp_o *= np.exp(G)[..., None]
    np.testing.assert_allclose(o, exp_o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(hT, np.exp(G[:, -1])[:, :, None, None] * h0, rtol=1e-13)


def test_state_orientation():
    """beta = 0, g = 0, q = e_i reads row i of the K-major state h0 [K, V]."""
    K, V = 4, 3
    h0 = np.arange(K * V, dtype=np.float64).reshape(1, 1, K, V) + 1.0
    q = np.eye(K)[None, :, None, :]
    k = np.zeros((1, K, 1, K))
    v = np.zeros((1, K, 1, V))
    g = np.zeros((1, K, 1))
    o, _ = oracle.forward(q, k, v, g, np.zeros((1, K, 1)), h0=h0)
    np.testing.assert_array_equal(o[0, :, 0], h0[0, 0])


def test_one_hot_keys_are_per_row_moving_averages():
    """One-hot keys: every row decays by alpha_t; the written row i_t becomes
    (1 - beta) * (its decayed value) + beta * v_t -- an exponential moving average."""
    rng = np.random.default_rng(3)
    K, V, S = 4, 3, 12
    idx = rng.integers(0, K, size=S)
    k = np.eye(K)[idx][None, :, None, :]
    q = rng.standard_normal((1, S, 1, K))
    v = rng.standard_normal((1, S, 1, V))
    g = -rng.uniform(0.0, 1.0, size=(1, S, 1))
    beta = rng.uniform(0.0, 1.0, size=(1, S, 1))
    h0 = rng.standard_normal((1, 1, K, V))
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    rows = h0[0, 0].copy()
    for t in range(S):
        rows = rows * np.exp(g[0, t, 0])
        i = idx[t]
        rows[i] = (1.0 - beta[0, t, 0]) * rows[i] + beta[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], q[0, t, 0] @ rows, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT[0, 0], rows, rtol=1e-12, atol=1e-14)


def test_retrieval_invariant_unit_keys():
    """With ||k_t|| = 1 and q_t = k_t, the read-out of the key just written is
    o_t = alpha_t (1 - beta_t) S_{t-1} k_t + beta_t v_t  (beta = 1 stores v_t exactly)."""
    rng = np.random.default_rng(4)
    B, S, H, K, V = 1, 10, 2, 6, 5
    k = rng.standard_normal((B, S, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, S, H, V))
    g = -rng.uniform(0.0, 2.0, size=(B, S, H))
    beta = rng.uniform(0.0, 1.0, size=(B, S, H))
    beta[:, ::3] = 1.0
    h0 = rng.standard_normal((B, H, K, V))
    o, _ = oracle.forward(k, k, v, g, beta, h0=h0)
    for t in range(S):
        _, h_prev = oracle.forward(k[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], h0=h0)
        for hh in range(H):
            read_prev = h_prev[0, hh].T @ k[0, t, hh]
            want = np.exp(g[0, t, hh]) * (1 - beta[0, t, hh]) * read_prev + beta[0, t, hh] * v[0, t, hh]
            np.testing.assert_allclose(o[0, t, hh], want, rtol=1e-11, atol=1e-12)
            if beta[0, t, hh] == 1.0:
                np.testing.assert_allclose(o[0, t, hh], v[0, t, hh], rtol=1e-11, atol=1e-12)


def test_scalar_key_closed_form():
    """K = 1: h_t = a_t h_{t-1} + beta_t k_t v_t with a_t = alpha_t (1 - beta_t k_t^2),
    so h_T = (prod a) h0 + sum_t (prod_{s>t} a_s) beta_t k_t v_t."""
    rng = np.random.default_rng(5)
    S, V = 15, 3
    k = rng.standard_normal((1, S, 1, 1)) * 0.7
    q = rng.standard_normal((1, S, 1, 1))
    v = rng.standard_normal((1, S, 1, V))
    g = -rng.uniform(0.0, 1.0, size=(1, S, 1))
    beta = rng.uniform(0.0, 1.0, size=(1, S, 1))
    h0 = rng.standard_normal((1, 1, 1, V))
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    a = np.exp(g[0, :, 0]) * (1 - beta[0, :, 0] * k[0, :, 0, 0] ** 2)
    b = (beta[0, :, 0] * k[0, :, 0, 0])[:, None] * v[0, :, 0]
    for t in range(S):
        tail = np.array([np.prod(a[s + 1:t + 1]) for s in range(t + 1)])
        h_t = np.prod(a[:t + 1]) * h0[0, 0, 0] + (tail[:, None] * b[:t + 1]).sum(0)
        np.testing.assert_allclose(o[0, t, 0], q[0, t, 0, 0] * h_t, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT[0, 0, 0], h_t, rtol=1e-12)


def test_affine_in_state_and_values():
    """The map (h0, v) -> (o, h_T) is linear for fixed q, k, g, beta
    (the affine chunk form h_out = M h + U with U linear in v)."""
    q, k, v, g, beta, h0 = _rand(6)
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    o1, h1 = oracle.forward(q, k, v, g, beta, h0=np.zeros_like(h0))
    o2, h2 = oracle.forward(q, k, np.zeros_like(v), g, beta, h0=h0)
    np.testing.assert_allclose(o, o1 + o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT, h1 + h2, rtol=1e-12, atol=1e-14)
    o3, h3 = oracle.forward(q, k, 2.5 * v, g, beta, h0=2.5 * h0)
    np.testing.assert_allclose(o3, 2.5 * o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h3, 2.5 * hT, rtol=1e-12, atol=1e-14)


def test_padding_is_bit_exact_noop():
    """Tokens with g = 0 and q = k = v = 0 are the identity (MaxText PR, section
    'Implementation': padded positions are a no-op for the recurrence)."""
    q, k, v, g, beta, h0 = _rand(7, S=8)
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    ins = [0, 3, 3, 8]      # insert pads before tokens 0, 3, 3 and at the end
    qp, kp, vp, gp, bp = (np.insert(a, ins, 0.0, axis=1) for a in (q, k, v, g, beta))
    bp[:, [0, 4, 5, 11]] = 0.7                  # beta of a pad is arbitrary
    op, hTp = oracle.forward(qp, kp, vp, gp, bp, h0=h0)
    real = np.delete(np.arange(op.shape[1]), [0, 4, 5, 11])
    np.testing.assert_array_equal(op[:, real], o)
    np.testing.assert_array_equal(hTp, hT)
    assert not op[:, [0, 4, 5, 11]].any()       # q = 0 reads nothing at a pad


@pytest.mark.parametrize("C", [1, 3, 4, 16, 64])
@pytest.mark.parametrize("decay", ["config", "slow"])
def test_chunked_form_matches_recurrence(C, decay):
    """The chunked WY algorithm (a different algorithm: triangular solves and
    chunk-level products) reproduces the token recurrence, with ragged tails."""
    q, k, v, g, beta, h0 = _rand(8, B=2, S=37, H=2, K=6, V=5, decay=decay)
    o_r, h_r = oracle.forward(q, k, v, g, beta, h0=h0)
    o_c, h_c = oracle.chunked_forward(q, k, v, g, beta, C, h0=h0)
    scale_o, scale_h = np.max(np.abs(o_r)), np.max(np.abs(h_r))
    assert np.max(np.abs(o_c - o_r)) <= 1e-12 * scale_o
    assert np.max(np.abs(h_c - h_r)) <= 1e-12 * scale_h


def test_chunked_form_at_head_dim_128():
    x = make_inputs(9, 1, 130, 1, 128, 128, 64, "bf16", 0.02, "config")
    o_r, h_r = oracle.forward(x.q, x.k, x.v, x.g, x.beta, h0=x.h0)
    o_c, h_c = oracle.chunked_forward(x.q, x.k, x.v, x.g, x.beta, 64, h0=x.h0)
    assert np.max(np.abs(o_c - o_r)) <= 1e-12 * np.max(np.abs(o_r))
    assert np.max(np.abs(h_c - h_r)) <= 1e-12 * np.max(np.abs(h_r))


def test_wy_factors_special_cases():
    """C = 1 makes T = I: w = beta exp(g) k and u = beta v.  beta = 0 gives w = u = 0."""
    q, k, v, g, beta, h0 = _rand(10, S=7)
    w, u = oracle.chunk_wy(k, v, g, beta, 1)
    np.testing.assert_allclose(w[:, :, :, 0], (beta * np.exp(g))[..., None] * k, rtol=1e-14)
    np.testing.assert_allclose(u[:, :, :, 0], beta[..., None] * v, rtol=1e-14)
    w0, u0 = oracle.chunk_wy(k, v, g, np.zeros_like(beta), 4)
    assert not w0.any() and not u0.any()


def test_wy_delta_rows_match_recurrence():
    """delta = u - w h0 of the first chunk equals the recurrence's per-token
    delta_t = beta_t (v_t - (alpha_t h_{t-1})^T k_t), read off as
    delta_t = (h_t - alpha_t h_{t-1})^T k_t / ||k_t||^2."""
    q, k, v, g, beta, h0 = _rand(11, B=1, S=6, H=1, K=5, V=4)
    w, u = oracle.chunk_wy(k, v, g, beta, 6)
    delta = u[0, 0, 0] - w[0, 0, 0] @ h0[0, 0]
    h_prev = h0[0, 0].astype(np.float64)
    for t in range(6):
        _, h_t = oracle.forward(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1],
                                beta[:, :t + 1], h0=h0)
        kt = k[0, t, 0].astype(np.float64)
        d_t = (h_t[0, 0] - np.exp(g[0, t, 0]) * h_prev).T @ kt / (kt @ kt)
        np.testing.assert_allclose(delta[t], d_t, rtol=1e-10, atol=1e-12)
        h_prev = h_t[0, 0]


def test_transition_pair_closed_forms():
    """beta = 0: M = exp(sum g) I.  Orthonormal keys written once each:
    M = (prod alpha)(I - sum_t beta_t k_t k_t^T)."""
    rng = np.random.default_rng(12)
    K, V, S = 6, 3, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm[:, :S].T[None, :, None, :]
    v = rng.standard_normal((1, S, 1, V))
    g = -rng.uniform(0, 1, size=(1, S, 1))
    beta = rng.uniform(0, 1, size=(1, S, 1))
    M, _ = oracle.transition_pair(k, v, g, beta)
    want = np.exp(g.sum()) * (np.eye(K) - sum(beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0])
                                              for t in range(S)))
    np.testing.assert_allclose(M[0, 0], want, rtol=1e-12, atol=1e-14)
    M0, _ = oracle.transition_pair(k, v, g, np.zeros_like(beta))
    np.testing.assert_allclose(M0[0, 0], np.exp(g.sum()) * np.eye(K), rtol=1e-13)


@pytest.mark.parametrize("decay", ["config", "slow"])
def test_transition_pair_is_the_affine_map(decay):
    """h_T(h0) = M h0 + U for an arbitrary h0 (M not transposed, U the zero-state end)."""
    q, k, v, g, beta, h0 = _rand(13, decay=decay)
    M, U = oracle.transition_pair(k, v, g, beta)
    _, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    np.testing.assert_allclose(hT, M @ h0 + U, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("C", [1, 4, 8])
def test_lowrank_composition_matches_transition(C):
    """Chunk-wise low-rank composition M <- gamma M - k_tilde^T (w M) (MaxText PR,
    section 'Implementation') gives the same (M, U) as the recurrence."""
    q, k, v, g, beta, h0 = _rand(14, S=21, decay="slow")
    M, U = oracle.transition_pair(k, v, g, beta)
    M2, U2 = oracle.lowrank_segment_pair(k, v, g, beta, C)
    np.testing.assert_allclose(M2, M, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(U2, U, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("cuts", [[0, 8], [0, 4, 12], [0, 4, 8, 16, 20]])
def test_segment_scan_reproduces_monolithic(cuts):
    """Associativity: per-segment (M_r, U_r) stitched by the exclusive scan give
    the monolithic state entering every segment and the final state."""
    q, k, v, g, beta, h0 = _rand(15, S=24, decay="slow")
    ends = cuts[1:] + [24]
    pairs = [oracle.transition_pair(k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b])
             for a, b in zip(cuts, ends)]
    M = np.stack([p[0] for p in pairs])
    U = np.stack([p[1] for p in pairs])
    h_in, h_fin = oracle.exclusive_scan(M, U, h0)
    _, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    np.testing.assert_allclose(h_fin, hT, rtol=1e-12, atol=1e-14)
    for r, a in enumerate(cuts):
        _, h_a = oracle.forward(q[:, :a], k[:, :a], v[:, :a], g[:, :a], beta[:, :a], h0=h0)
        np.testing.assert_allclose(h_in[r], h_a, rtol=1e-12, atol=1e-14)


def test_negative_controls_fail():
    """Plausible mistakes in the segment stitching must be caught: permuted
    segments, M replaced by I or 0, M transposed (slow decay keeps M alive)."""
    q, k, v, g, beta, h0 = _rand(16, S=24, decay="slow")
    cuts = [0, 8, 16]
    pairs = [oracle.transition_pair(k[:, a:a + 8], v[:, a:a + 8], g[:, a:a + 8], beta[:, a:a + 8])
             for a in cuts]
    M = np.stack([p[0] for p in pairs])
    U = np.stack([p[1] for p in pairs])
    _, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    scale = np.max(np.abs(hT))
    bad = {
        "permuted": oracle.exclusive_scan(M[[1, 0, 2]], U[[1, 0, 2]], h0)[1],
        "M=I": oracle.exclusive_scan(np.broadcast_to(np.eye(M.shape[-1]), M.shape), U, h0)[1],
        "M=0": oracle.exclusive_scan(np.zeros_like(M), U, h0)[1],
        "M^T": oracle.exclusive_scan(np.swapaxes(M, -1, -2), U, h0)[1],
    }
    for name, h in bad.items():
        assert np.max(np.abs(h - hT)) > 1e-3 * scale, name


def test_packed_equals_per_sequence():
    x = make_packed_inputs(17, 3, 70, 2, 5, 4, 8, "f32", 0.3, median=20)
    o, hT = oracle.forward_packed(x.cu_seqlens, x.q[0], x.k[0], x.v[0], x.g[0], x.beta[0], h0=x.h0)
    for n in range(3):
        a, b = x.cu_seqlens[n], x.cu_seqlens[n + 1]
        o_n, h_n = oracle.forward(x.q[:, a:b], x.k[:, a:b], x.v[:, a:b], x.g[:, a:b],
                                  x.beta[:, a:b], h0=x.h0[n:n + 1])
        np.testing.assert_array_equal(o[a:b], o_n[0])
        np.testing.assert_array_equal(hT[n], h_n[0])


def test_decode_steps_equal_forward():
    d = make_decode_inputs(18, 3, 2, 5, 4, 6, dtype="f32", state_std=0.5)
    state = d.state0.astype(np.float64)
    outs = []
    for t in range(6):
        o, state = oracle.decode_step(d.q[t], d.k[t], d.v[t], d.g[t], d.beta[t], state)
        outs.append(o)
    sw = lambda a: np.swapaxes(a, 0, 1)  # [steps,B,...] -> [B,steps,...]
    o_f, h_f = oracle.forward(sw(d.q), sw(d.k), sw(d.v), sw(d.g), sw(d.beta), h0=d.state0)
    np.testing.assert_allclose(np.stack(outs, 1), o_f, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(state, h_f, rtol=1e-13, atol=1e-15)


def _exact_forward(q, k, v, alpha, beta, h0):
    """Exact rational arithmetic, one chain; alpha given directly (no exp)."""
    S, K = len(k), len(k[0])
    V = len(v[0])
    h = [[Fraction(x) for x in row] for row in h0]
    o = []
    for t in range(S):
        h = [[alpha[t] * x for x in row] for row in h]
        d = [beta[t] * (v[t][j] - sum(h[i][j] * k[t][i] for i in range(K))) for j in range(V)]
        h = [[h[i][j] + k[t][i] * d[j] for j in range(V)] for i in range(K)]
        o.append([sum(h[i][j] * q[t][i] for i in range(K)) for j in range(V)])
    return o, h


def test_c_oracle_indexing_against_exact_arithmetic():
    """Multi-batch, multi-head tiny case against exact rationals: catches stride
    and indexing mistakes in the C loops (alpha = exp(g) taken from the same
    fp64 exp, converted exactly)."""
    rng = np.random.default_rng(19)
    B, S, H, K, V = 2, 5, 3, 3, 2
    q, k, v = (rng.integers(-4, 5, size=s).astype(np.float64) / 4
               for s in [(B, S, H, K), (B, S, H, K), (B, S, H, V)])
    g = -rng.integers(0, 4, size=(B, S, H)).astype(np.float64) / 8
    beta = rng.integers(0, 5, size=(B, S, H)).astype(np.float64) / 4
    h0 = rng.integers(-4, 5, size=(B, H, K, V)).astype(np.float64) / 2
    o, hT = oracle.forward(q, k, v, g, beta, h0=h0)
    F = lambda a: [[Fraction(float(x)) for x in row] for row in a]
    for b in range(B):
        for hh in range(H):
            alpha = [Fraction(float(np.exp(g[b, t, hh]))) for t in range(S)]
            oe, he = _exact_forward(F(q[b, :, hh]), F(k[b, :, hh]), F(v[b, :, hh]), alpha,
                                    [Fraction(float(x)) for x in beta[b, :, hh]], F(h0[b, hh]))
            np.testing.assert_allclose(o[b, :, hh], np.array(oe, dtype=np.float64), rtol=1e-14,
                                       atol=1e-15)
            np.testing.assert_allclose(hT[b, hh], np.array(he, dtype=np.float64), rtol=1e-14,
                                       atol=1e-15)


def test_grouped_key_heads_order_and_meaning():
    """Grouped key heads ("RFC(qwen35): TP Phase 2", section "Partition
    Contract"; grouped order from the Ulysses page's examples at cp = 4 and 8):
    each key head serves consecutive value heads, [kv0, kv0, kv1, kv1] and not
    the tiled [kv0, kv1, kv0, kv1]; one key head per value head is the identity;
    two value heads reading one key head with equal v, g, beta give equal results."""
    labels = np.arange(2).reshape(1, 2, 1)
    assert oracle.expand_key_heads(labels, 4)[0, :, 0].tolist() == [0, 0, 1, 1]
    assert oracle.expand_key_heads(labels, 8)[0, :, 0].tolist() == [0] * 4 + [1] * 4
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((1, 20, 2, 4)), rng.standard_normal((1, 20, 2, 4))
    assert np.array_equal(oracle.expand_key_heads(q, 2), q)
    with pytest.raises(ValueError):
        oracle.expand_key_heads(q, 3)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = np.repeat(rng.standard_normal((1, 20, 1, 4)), 4, axis=2)
    g = np.repeat(-np.abs(rng.standard_normal((1, 20, 1))), 4, axis=2) * 0.1
    beta = np.repeat(rng.random((1, 20, 1)), 4, axis=2)
    o, h = oracle.forward(oracle.expand_key_heads(q, 4), oracle.expand_key_heads(k, 4), v, g, beta)
    assert np.array_equal(o[:, :, 0], o[:, :, 1]) and np.array_equal(o[:, :, 2], o[:, :, 3])
    assert not np.allclose(o[:, :, 1], o[:, :, 2])
    assert np.array_equal(h[:, 0], h[:, 1])


# ---- the steps beside the core: depthwise causal conv and gated RMSNorm -------------------

def _conv_case(seed, T=11, D=6, W=4):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, D)), rng.standard_normal((D, W)), rng.standard_normal((D, W - 1))


def test_causal_conv_identity_and_shift_taps():
    """Taps (0,..,0,1) pass x through; taps (1,0,..,0) delay it by W-1 tokens,
    the first W-1 outputs coming from the state; the new state is the last W-1
    positions."""
    x, _, st = _conv_case(1)
    ident = np.zeros((6, 4)); ident[:, 3] = 1
    y, s2 = oracle.causal_conv1d(x, ident, st, activation="none")
    assert np.array_equal(y, x) and np.array_equal(s2, x[-3:].T)
    shift = np.zeros((6, 4)); shift[:, 0] = 1
    y, _ = oracle.causal_conv1d(x, shift, st, activation="none")
    assert np.array_equal(y[:3], st.T) and np.array_equal(y[3:], x[:-3])
    y0, _ = oracle.causal_conv1d(x, shift, None, activation="none")
    assert np.array_equal(y0[:3], np.zeros((3, 6)))


def test_causal_conv_matches_numpy_convolve():
    """Each channel against numpy's full convolution with the reversed taps
    (a library routine), state prepended."""
    x, w, st = _conv_case(2)
    y, _ = oracle.causal_conv1d(x, w, st, activation="none")
    for c in range(6):
        full = np.convolve(np.concatenate([st[c], x[:, c]]), w[c, ::-1], mode="full")
        np.testing.assert_allclose(y[:, c], full[3:3 + 11], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("cut", [0, 1, 2, 3, 7, 11])
def test_causal_conv_streams_through_its_state(cut):
    """Convolving [a | b] equals convolving a, then b from a's final state, also
    when a is shorter than the W-1 tokens the state holds (decode steps)."""
    x, w, st = _conv_case(3)
    y, s_end = oracle.causal_conv1d(x, w, st)
    ya, sa = oracle.causal_conv1d(x[:cut], w, st)
    yb, sb = oracle.causal_conv1d(x[cut:], w, sa)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(sb, s_end, rtol=0, atol=0)


def test_silu_and_gated_rmsnorm_closed_forms():
    """SiLU(u) = u * sigmoid(u) (scipy's expit); RMSNorm of c*1 is sign(c) as
    eps -> 0; it is invariant to positive scaling; with eps = 0 it equals
    o * sqrt(V) / ||o||; the gate multiplies elementwise by SiLU(z)."""
    from scipy.special import expit
    u = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(oracle.silu(u), u * expit(u), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    V = 8
    one = np.ones(V)
    np.testing.assert_allclose(oracle.gated_rmsnorm(-3.0 * one, one, eps=0.0), -one, rtol=1e-15)
    rng = np.random.default_rng(4)
    o, w, z = rng.standard_normal((5, V)), rng.standard_normal(V), rng.standard_normal((5, V))
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * o, w, eps=0.0), oracle.gated_rmsnorm(o, w, eps=0.0),
                               rtol=1e-13)
    ref = o * np.sqrt(V) / np.linalg.norm(o, axis=-1, keepdims=True) * w
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, w, eps=0.0), ref, rtol=1e-13)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, w, z, eps=0.0), ref * z * expit(z), rtol=1e-13)


@pytest.mark.parametrize("L", [1, 5, 16])
def test_chunk_transition_is_one_chunks_affine_map(L):
    """(M_c, U_c) of one chunk from the chunk form (gamma I - k_tilde^T w,
    k_tilde^T u) equals the pair the recurrence defines over the same tokens:
    M by running it from the identity with v = 0, U from the zero state."""
    rng = np.random.default_rng(40 + L)
    K, V = 5, 3
    k = rng.standard_normal((L, K)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, V))
    g = -np.log1p(np.exp(rng.standard_normal(L) - 2.0))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    Mc, Uc = oracle.chunk_transition(k, v, g, beta)
    M, U = oracle.transition_pair(k[None, :, None], v[None, :, None], g[None, :, None], beta[None, :, None])
    np.testing.assert_allclose(Mc, M[0, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Uc, U[0, 0], rtol=1e-12, atol=1e-14)
    # and a state pushed through it equals the recurrence's end state
    h0 = rng.standard_normal((K, V))
    _, hT = oracle.forward(np.zeros((1, L, 1, K)), k[None, :, None], v[None, :, None], g[None, :, None],
                           beta[None, :, None], h0=h0[None, None])
    np.testing.assert_allclose(Mc @ h0 + Uc, hT[0, 0], rtol=1e-12, atol=1e-14)


def test_causal_conv_packed_equals_per_sequence():
    """The packed conv is the per-sequence conv laid end to end: every
    sequence, including empty ones and ones shorter than the W - 1 state
    positions, starts from its own state row and leaves its own final state
    (bit-exact, the same fp64 operations in the same order)."""
    rng = np.random.default_rng(7)
    D, W = 6, 4
    lens = [5, 0, 1, 2, 9, 0, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = rng.standard_normal((int(cu[-1]), D))
    w = rng.standard_normal((D, W))
    st = rng.standard_normal((len(lens), D, W - 1))
    for act in ("silu", "none"):
        y, s = oracle.causal_conv1d_packed(x, w, cu, st, activation=act)
        for n in range(len(lens)):
            a, b = int(cu[n]), int(cu[n + 1])
            yn, sn = oracle.causal_conv1d(x[a:b], w, st[n], activation=act)
            assert np.array_equal(y[a:b], yn) and np.array_equal(s[n], sn)
        # an empty sequence hands its state through unchanged; a one-token
        # sequence shifts it by one position
        assert np.array_equal(s[1], st[1]) and np.array_equal(s[5], st[5])
        assert np.array_equal(s[2][:, :-1], st[2][:, 1:]) and np.array_equal(s[2][:, -1], x[cu[2]])
        # the first output of a sequence reads its own state, not the tokens
        # of the sequence before it (taps (1, 0, 0, 0) pick the oldest position)
        shift = np.zeros((D, W)); shift[:, 0] = 1
        ys, _ = oracle.causal_conv1d_packed(x, shift, cu, st, activation="none")
        assert np.array_equal(ys[cu[4]], st[4][:, 0])
    # no state: zeros before every sequence start
    y0, s0 = oracle.causal_conv1d_packed(x, w, cu, None, activation="none")
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        yn, sn = oracle.causal_conv1d(x[a:b], w, None, activation="none")
        assert np.array_equal(y0[a:b], yn) and np.array_equal(s0[n], sn)
    assert np.array_equal(s0[1], np.zeros((D, W - 1)))
