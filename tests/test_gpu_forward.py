"""GPU parity of the chunked forward (prepare, scan, segment pass) against the
fp64 oracle, through the C ABI.  Bound: normwise relative error <= 1e-4 for
fp32 inputs and <= 2e-2 for bf16 inputs, on the outputs and the final states."""
import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_gdn_amd as gdn
from workloads import make_inputs, make_packed_inputs, workload
from gpu_util import (TOL, DEV, say, device_inputs, oracle_forward, rel_err, run_forward, tdt,
                      to_dev, check_forward, slice_err)

pytestmark = pytest.mark.gpu


check = check_forward


# ---- tiny fp32 workload (B1 H2 S256 K=V=32 C16) -------------------------------------------

@pytest.mark.parametrize("n_segments", [1, 2, 4])
@pytest.mark.parametrize("reuse_wy", [False, True])
def test_tiny_f32(n_segments, reuse_wy):
    x = workload(0)
    o, hT = run_forward(x, n_segments=n_segments, reuse_wy=reuse_wy)
    o_ref, h_ref = oracle_forward(x)
    check(x, o, hT, o_ref, h_ref, what=f"R={n_segments} wy={reuse_wy}")


@pytest.mark.parametrize("decay", ["slow", "none"])
def test_tiny_f32_slow_decay_segments(decay):
    """Slow decay keeps M alive across segments, so a wrong M would show."""
    x = workload(0, decay=decay)
    x.h0 = np.random.default_rng(5).standard_normal((1, 2, 32, 32)).astype(np.float32) * 0.1
    o_ref, h_ref = oracle_forward(x)
    for R in (1, 4, 16):
        o, hT = run_forward(x, n_segments=R)
        check(x, o, hT, o_ref, h_ref, what=f"{decay} R={R}")


def test_tiny_f32_segment_matches_monolithic_closely():
    """fp32 segment pass vs monolithic pass: the MaxText PR reports f32 parity of
    9.9e-8 (output) and 1.4e-7 (final state) at cp=4 ('Measured results').  The
    bound here is 1e-6, a few times that level (a different summation order
    over 64 fp32 products per entry); the achieved figures are printed."""
    x = workload(0, decay="slow")
    o1, h1 = run_forward(x, n_segments=1)
    for R in (2, 4):
        oR, hR = run_forward(x, n_segments=R)
        eo, eh = rel_err(oR, o1), rel_err(hR, h1)
        say(f"  fp32 segments R={R} vs monolithic: err(o)={eo:.2e} err(hT)={eh:.2e}")
        assert eo < 1e-6 and eh < 1e-6


# ---- bf16 at head dim 128 -------------------------------------------------------------------

def test_seq4k_bf16():
    x = workload(1)
    o, hT = run_forward(x)
    o_ref, h_ref = oracle_forward(x)
    check(x, o, hT, o_ref, h_ref)


@pytest.mark.parametrize("R", [2, 4])
def test_seq4k_bf16_segments_slow_decay(R):
    x = workload(1, H=4, decay="slow")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=R)
    check(x, o, hT, o_ref, h_ref, what=f"slow R={R}")


@pytest.mark.parametrize("schedule", ["auto", "plain"])
@pytest.mark.parametrize("R", [2, 3, 4])
def test_seq4k_bf16_segment_schedules(schedule, R):
    """Both schedules of the segment pass (overlapped: segment 0 emitted from h0
    beside the carrying pass of the middle segments; plain: carrying pass over
    every segment), slow decay so M matters."""
    x = workload(1, H=4, decay="slow")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=R, schedule=schedule)
    check(x, o, hT, o_ref, h_ref, what=f"R={R} schedule={schedule}")


@pytest.mark.parametrize("schedule", ["auto", "plain"])
def test_tiny_f32_segment_schedules_uneven(schedule):
    """fp32 vector-ALU path, explicit uneven segment starts, both schedules."""
    x = workload(0, decay="slow")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=3, seg_starts=[0, 48, 208], schedule=schedule)
    check(x, o, hT, o_ref, h_ref, what=f"starts 0,48,208 schedule={schedule}")


def test_seq4k_bf16_reuse_wy():
    x = workload(1, H=4)
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=2, reuse_wy=True)
    check(x, o, hT, o_ref, h_ref, what="wy reused")


def test_seq4k_bf16_reuse_wy_slow_decay_segments():
    """WY factors reused by the carrying and emitting passes, with slow decay so
    the segment transitions M are far from zero."""
    x = workload(1, H=4, decay="slow")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=4, reuse_wy=True)
    check(x, o, hT, o_ref, h_ref, what="wy reused, 4 segments")


def test_packed_ragged_reuse_wy():
    """WY factors reused on unpadded packed sequences at K = V = 128."""
    rng = np.random.default_rng(13)
    x = make_inputs(13, 1, 500, 2, 128, 128, 64, "bf16", 0.0, name="packed-ragged-wy")
    x.cu_seqlens = np.array([0, 100, 100, 231, 420, 500], dtype=np.int32)
    x.h0 = rng.standard_normal((5, 2, 128, 128)).astype(np.float32) * 0.02
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, reuse_wy=True)
    check(x, o[0], hT, o_ref, h_ref, what="wy reused")


def test_seq64k_four_segments_sampled_heads():
    """The 64k-token, 32-head, 4-segment workload in the launch configuration the
    benchmark times; the oracle recomputes two sampled heads in full."""
    x = workload(2)
    o, hT = run_forward(x, n_segments=4)
    heads = [0, 29]
    o_ref, h_ref = oracle_forward(x, heads=heads)
    check(x, o[:, :, heads], hT[:, heads], o_ref, h_ref, what=f"heads {heads}")
    o1, h1 = run_forward(x, n_segments=1)
    assert rel_err(o, o1) <= TOL["bf16"] and rel_err(hT, h1) <= TOL["bf16"]


def test_packed_varlen_sampled_heads():
    x = workload(3)
    o, hT = run_forward(x)
    heads = [3, 17, 31]
    o_ref, h_ref = oracle_forward(x, heads=heads)
    check(x, o[0][:, heads], hT[:, heads], o_ref, h_ref, what=f"heads {heads}")
    # padded positions produce zero output
    lens = x.meta["lengths"]
    for n, L in enumerate(lens):
        a, b = int(x.cu_seqlens[n]) + L, int(x.cu_seqlens[n + 1])
        assert not np.any(o[0, a:b])


# ---- edge cases -----------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1, 15, 16, 17, 100, 250])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_lengths_small(S, dtype):
    x = make_inputs(100 + S, 2, S, 3, 32, 32, 16, dtype, 0.3, "config", name=f"ragged{S}")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x)
    check(x, o, hT, o_ref, h_ref, what=f"S={S}")


# 1 to 5 chunks: the emitting loader runs its chunks in pairs with an odd one
# after, and keeps two chunks of k rows in flight (the last chunk reloaded past
# the end)
@pytest.mark.parametrize("S", [1, 63, 65, 128, 129, 192, 200, 257])
def test_ragged_lengths_128(S):
    x = make_inputs(200 + S, 2, S, 2, 128, 128, 64, "bf16", 0.02, "config", name=f"ragged{S}")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x)
    check(x, o, hT, o_ref, h_ref, what=f"S={S}")


def test_empty_sequence_returns_initial_state():
    x = make_inputs(7, 2, 0, 2, 32, 32, 16, "f32", 0.5, name="empty")
    o, hT = run_forward(x)
    assert o.shape == (2, 0, 2, 32)
    np.testing.assert_array_equal(hT, x.h0)


def test_packed_ragged_and_empty_sequences():
    """Unpadded packed sequences (lengths not multiples of C, one empty)."""
    rng = np.random.default_rng(11)
    base = make_inputs(11, 1, 300, 2, 32, 32, 16, "bf16", 0.0, name="packed-ragged")
    cu = np.array([0, 37, 37, 160, 161, 300], dtype=np.int32)
    base.cu_seqlens = cu
    base.h0 = rng.standard_normal((5, 2, 32, 32)).astype(np.float32) * 0.1
    o_ref, h_ref = oracle_forward(base)
    o, hT = run_forward(base)
    check(base, o[0], hT, o_ref, h_ref, what="cu=" + ",".join(map(str, cu)))
    np.testing.assert_array_equal(hT[1], base.h0[1])


def test_explicit_segment_starts_uneven():
    x = make_inputs(12, 1, 500, 2, 32, 32, 16, "f32", 0.3, "slow", name="uneven-seg")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=3, seg_starts=[0, 16, 400])
    check(x, o, hT, o_ref, h_ref, what="seg 0,16,400")


def test_unordered_segments_raise_and_write_nothing():
    x = workload(0)
    d = device_inputs(x)
    o = torch.full((1, 256, 2, 32), 7.0, device=DEV)
    with pytest.raises(ValueError, match="contiguous and in order"):
        gdn.scan_emit(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=16, n_segments=3,
                      seg_starts=[0, 64, 32], out=o)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)


def test_state_in_place_continuation():
    """Prefill [0, s) then [s, S) with the carried state, h_out aliasing h_in,
    equals one pass over [0, S)."""
    from chunked_gated_delta_gdn_amd import binding as b
    x = workload(1, H=2, S=1000)
    d = device_inputs(x)
    state = d["h0"].clone()
    o = torch.empty_like(d["v"])
    stream = torch.cuda.current_stream().cuda_stream
    for a, e in [(0, 448), (448, 1000)]:
        qs, ks, vs, gs, bs = (t[:, a:e].contiguous() for t in
                              (d["q"], d["k"], d["v"], d["g"], d["beta"]))
        part = torch.empty_like(vs)
        p = gdn.problem_for(ks, vs, 64)
        b.gdn_scan(p, b.GDN_SCAN_EMIT, qs.data_ptr(), ks.data_ptr(), vs.data_ptr(),
                   gs.data_ptr(), bs.data_ptr(), None, 0, state.data_ptr(), part.data_ptr(),
                   state.data_ptr(), None, None, stream)
        o[:, a:e] = part
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_forward(x)
    check(x, o.float().cpu().numpy(), state.cpu().numpy(), o_ref, h_ref,
          what="two-part prefill")


def test_deterministic():
    x = workload(1, H=4, S=1024)
    o1, h1 = run_forward(x, n_segments=2)
    o2, h2 = run_forward(x, n_segments=2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)


# ---- the individual entry points ------------------------------------------------------------

@pytest.mark.parametrize("wl,tol", [(0, 1e-4), (1, 2e-2)])
def test_chunk_prepare_wy_factors(wl, tol):
    x = workload(wl, H=2, S=300)
    d = device_inputs(x)
    wy = gdn.chunk_prepare(d["k"], d["v"], d["g"], d["beta"], chunk_size=x.C)
    w, u = gdn.split_wy(wy, d["k"], d["v"], x.C)
    w_ref, u_ref = oracle.chunk_wy(x.k, x.v, x.g, x.beta, x.C)     # [B,Nc,H,C,*]
    w = w.float().cpu().numpy().reshape(w_ref.shape)
    u = u.float().cpu().numpy().reshape(u_ref.shape)
    ew, eu = rel_err(w, w_ref), rel_err(u, u_ref)
    say(f"  wy {x.name}: err(w)={ew:.3e} err(u)={eu:.3e}")
    assert ew <= tol and eu <= tol


def test_chunk_prepare_wy_seq4k():
    """WY factors of the whole 4k-token, 16-head workload (the matrix-core
    preparation path at full size)."""
    x = workload(1)
    d = device_inputs(x)
    wy = gdn.chunk_prepare(d["k"], d["v"], d["g"], d["beta"], chunk_size=x.C)
    w, u = gdn.split_wy(wy, d["k"], d["v"], x.C)
    w_ref, u_ref = oracle.chunk_wy(x.k, x.v, x.g, x.beta, x.C)
    w = w.float().cpu().numpy().reshape(w_ref.shape)
    u = u.float().cpu().numpy().reshape(u_ref.shape)
    ew, eu = rel_err(w, w_ref), rel_err(u, u_ref)
    say(f"  wy {x.name}: err(w)={ew:.3e} err(u)={eu:.3e}")
    assert ew <= TOL["bf16"] and eu <= TOL["bf16"]


def test_chunk_prepare_packed_ragged_and_empty():
    """WY factors of unpadded packed sequences (ragged tails, one empty), in
    global chunk order, at K = V = 128."""
    x = make_inputs(12, 1, 400, 2, 128, 128, 64, "bf16", 0.0, name="prep-packed")
    cu = np.array([0, 70, 70, 200, 329, 400], dtype=np.int32)
    d = device_inputs(x)
    wy = gdn.chunk_prepare(d["k"], d["v"], d["g"], d["beta"], chunk_size=64, cu_seqlens=cu)
    w, u = gdn.split_wy(wy, d["k"], d["v"], 64)
    ws, us = [], []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        wr, ur = oracle.chunk_wy(x.k[:, a:b], x.v[:, a:b], x.g[:, a:b], x.beta[:, a:b], 64)
        ws.append(wr[0])
        us.append(ur[0])
    w_ref, u_ref = np.concatenate(ws), np.concatenate(us)
    assert w.shape == w_ref.shape and u.shape == u_ref.shape
    w, u = w.float().cpu().numpy(), u.float().cpu().numpy()
    ew, eu = rel_err(w, w_ref), rel_err(u, u_ref)
    say(f"  wy packed cu={cu.tolist()}: err(w)={ew:.3e} err(u)={eu:.3e}")
    assert ew <= TOL["bf16"] and eu <= TOL["bf16"]


@pytest.mark.parametrize("wl", [0, 1])
def test_carry_pairs_match_transition(wl):
    x = workload(wl, H=2, S=512, decay="slow")
    d = device_inputs(x)
    M, U = gdn.scan_carry(d["k"], d["v"], d["g"], d["beta"], chunk_size=x.C, n_segments=2)
    torch.cuda.synchronize()
    for r, (a, b) in enumerate([(0, 256), (256, 512)]):
        M_ref, U_ref = oracle.transition_pair(x.k[:, a:b], x.v[:, a:b], x.g[:, a:b],
                                              x.beta[:, a:b])
        em = rel_err(M[r].cpu().numpy(), M_ref)
        eu = rel_err(U[r].cpu().numpy(), U_ref)
        say(f"  carry {x.name} seg {r}: err(M)={em:.3e} err(U)={eu:.3e}")
        assert em <= TOL[x.dtype] and eu <= TOL[x.dtype]


@pytest.mark.parametrize("shape,B", [("f32", 1), ("bf16", 1), ("bf16", 2)])
def test_head_emit_carry_matches_separate_passes(shape, B):
    """GDN_SCAN_HEAD_EMIT_CARRY (one launch on the matrix-core path, two generic
    launches otherwise) against the emitting pass of segment 0 and the carrying
    pass of the rest, element for element, and segment 0's final state against
    the oracle.  Ragged last chunk, three segments, nonzero initial state."""
    K, C, dt = (32, 16, "f32") if shape == "f32" else (128, 64, "bf16")
    S = 5 * C + 9
    x = make_inputs(41, B, S, 2, K, K, C, dt, 0.02, decay="slow", name=f"head-{shape}-B{B}")
    d = device_inputs(x)
    R = 3
    bnd = gdn.segment_bounds(S, C, R)
    s1 = bnd[1]
    o, h1, M, U = gdn.scan_head_carry(d["q"], d["k"], d["v"], d["g"], d["beta"], h_in=d["h0"], chunk_size=C,
                                      n_segments=R)
    head = {n: d[n][:, :s1].contiguous() for n in ("q", "k", "v", "g", "beta")}
    tail = {n: d[n][:, s1:].contiguous() for n in ("k", "v", "g", "beta")}
    o_e, h1_e = gdn.scan_emit(head["q"], head["k"], head["v"], head["g"], head["beta"], h_in=d["h0"],
                              chunk_size=C)
    M_c, U_c = gdn.scan_carry(tail["k"], tail["v"], tail["g"], tail["beta"], chunk_size=C, n_segments=R - 1,
                              seg_starts=[b - s1 for b in bnd[1:R]])
    torch.cuda.synchronize()
    assert torch.equal(o[:, :s1], o_e)
    assert torch.equal(h1, h1_e)
    assert torch.equal(M, M_c) and torch.equal(U, U_c)
    _, h1_ref = oracle.forward(x.q[:, :s1], x.k[:, :s1], x.v[:, :s1], x.g[:, :s1], x.beta[:, :s1], h0=x.h0,
                               want_o=False)
    err = rel_err(h1.cpu().numpy(), h1_ref)
    say(f"  head emit + carry {shape} B={B}: err(h1)={err:.3e}")
    assert err <= TOL[dt]


def test_segment_compose_matches_oracle_scan():
    rng = np.random.default_rng(21)
    R, N, H, K, V = 5, 2, 3, 128, 128
    M = (rng.standard_normal((R, N, H, K, K)) / np.sqrt(K)).astype(np.float32)
    U = rng.standard_normal((R, N, H, K, V)).astype(np.float32)
    h0 = rng.standard_normal((N, H, K, V)).astype(np.float32)
    h_in, h_fin = gdn.segment_compose(to_dev(M), to_dev(U), to_dev(h0), want_final=True)
    torch.cuda.synchronize()
    ref_in, ref_fin = oracle.exclusive_scan(M, U, h0)
    assert rel_err(h_in.cpu().numpy(), ref_in) <= 1e-5
    assert rel_err(h_fin.cpu().numpy(), ref_fin) <= 1e-5


@pytest.mark.parametrize("R,K,with_h0,want_final", [(1, 128, False, False), (3, 128, False, True),
                                                     (2, 128, True, False), (4, 32, True, True)])
def test_segment_compose_variants(R, K, with_h0, want_final):
    """Single segment (no products), zero initial state, no final state, and the
    K = V = 32 shape, against the oracle's exclusive scan."""
    rng = np.random.default_rng(22 + R)
    N, H = 1, 4
    M = (rng.standard_normal((R, N, H, K, K)) / np.sqrt(K)).astype(np.float32)
    U = rng.standard_normal((R, N, H, K, K)).astype(np.float32)
    h0 = rng.standard_normal((N, H, K, K)).astype(np.float32) if with_h0 else None
    h_in, h_fin = gdn.segment_compose(to_dev(M), to_dev(U), to_dev(h0) if with_h0 else None,
                                      want_final=want_final)
    torch.cuda.synchronize()
    ref_in, ref_fin = oracle.exclusive_scan(M, U, h0)
    say(f"  compose R={R} K={K} h0={with_h0}: err(h_in)={rel_err(h_in.cpu().numpy(), ref_in):.3e}")
    assert rel_err(h_in.cpu().numpy(), ref_in) <= 1e-5
    if want_final:
        assert rel_err(h_fin.cpu().numpy(), ref_fin) <= 1e-5
    else:
        assert h_fin is None


# ---- limits and degenerate cases ------------------------------------------------------------

def test_packed_max_sequences():
    """GDN_MAX_SEQS (256) packed sequences of mixed lengths, some empty, some
    shorter than a chunk, at K = V = 128."""
    rng = np.random.default_rng(21)
    lens = rng.integers(0, 150, size=256)
    lens[::17] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(21, 1, int(cu[-1]), 2, 128, 128, 64, "bf16", 0.0, name="packed-256")
    x.cu_seqlens = cu
    x.h0 = rng.standard_normal((256, 2, 128, 128)).astype(np.float32) * 0.02
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x)
    check(x, o[0], hT, o_ref, h_ref, what=f"256 sequences, {int(cu[-1])} tokens")
    for n in np.nonzero(lens == 0)[0]:
        np.testing.assert_array_equal(hT[n], x.h0[n])


def test_too_many_sequences_rejected():
    x = make_inputs(22, 1, 257, 1, 32, 32, 16, "f32", 0.0)
    d = device_inputs(x)
    cu = np.arange(258, dtype=np.int32)
    with pytest.raises(ValueError):
        gdn.scan_emit(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=16, cu_seqlens=cu)


@pytest.mark.parametrize("schedule", ["auto", "plain"])
def test_max_segments(schedule):
    """GDN_MAX_SEGMENTS (64) one-chunk segments, slow decay."""
    x = make_inputs(23, 1, 64 * 64, 2, 128, 128, 64, "bf16", 0.02, decay="slow", name="64-segments")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=64, schedule=schedule)
    check(x, o, hT, o_ref, h_ref, what=f"R=64 schedule={schedule}")


def test_batch_of_two_with_segments():
    """B = 2 sequences, each cut into 3 segments (the plain schedule)."""
    x = make_inputs(24, 2, 1000, 2, 128, 128, 64, "bf16", 0.02, decay="slow", name="B2-segments")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=3)
    check(x, o, hT, o_ref, h_ref, what="B=2 R=3")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beta_zero_is_pure_decay(dtype):
    """beta = 0: the state only decays, o_t = exp(G_t) h0^T q_t (the closed form
    the oracle is pinned to)."""
    K = 32 if dtype == "f32" else 128
    C = 16 if dtype == "f32" else 64
    # slow decay: under the workload decay the state falls to ~1e-105 over 300
    # tokens, below fp32 range
    x = make_inputs(25, 1, 300, 2, K, K, C, dtype, 0.05, decay="slow", name="beta0")
    x.beta[:] = 0
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=2)
    check(x, o, hT, o_ref, h_ref, what="beta=0")
    G = np.cumsum(x.g[0].astype(np.float64), axis=0)           # [S,H]
    o_cf = np.exp(G)[:, :, None] * np.einsum("shk,hkv->shv", x.q[0].astype(np.float64), x.h0[0])
    assert rel_err(o[0], o_cf) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_segments", [1, 3])
def test_mixed_degenerate_tokens(dtype, n_segments):
    """Scattered degenerate tokens inside chunks: beta = 0 (no write; the
    matrix-core path folds beta in as the exponent -log2(beta) = +inf), g = 0
    (no decay), g = -40 (a hard reset of the state), and zero keys or zero
    queries.  Nothing may turn into NaN and the result follows the oracle."""
    K = 32 if dtype == "f32" else 128
    C = 16 if dtype == "f32" else 64
    S = 5 * C + 7
    x = make_inputs(26, 1, S, 2, K, K, C, dtype, 0.05, decay="slow", name="degenerate")
    rng = np.random.default_rng(26)
    pick = lambda frac: rng.random((1, S, 2)) < frac
    x.beta[pick(0.2)] = 0.0
    x.g[pick(0.2)] = 0.0
    x.g[pick(0.03)] = -40.0
    x.k[pick(0.05)] = 0
    x.q[pick(0.05)] = 0
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=n_segments)
    check(x, o, hT, o_ref, h_ref, what=f"degenerate tokens R={n_segments}")


def test_no_decay_4k():
    """g = 0 (alpha = 1) over 4k tokens, 4 segments: no forgetting at all."""
    x = workload(1, H=4, decay="none")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=4)
    check(x, o, hT, o_ref, h_ref, what="g=0 R=4")


# ---- the overwrite table at full size, and gates outside the usual ranges --------------------

def _overwrite_inputs(S=512, H=2, seed=21):
    """One-hot keys and queries, beta = 1, g = 0 (the textbook overwrite
    table: writing key e_i replaces row i of the state by v), at K = V = 128,
    C = 64, bf16.  Head h's first chunk writes one key 64 times; the next two
    chunks write runs of 1 to 24 tokens over four keys; the rest random keys.
    Repeated keys make A0 diag(beta) an all-ones block, the hardest case for
    the triangular inverse (its powers reach binomial sizes)."""
    rng = np.random.default_rng(seed)
    K = V = 128
    idx = np.zeros((S, H), dtype=np.int64)
    for h in range(H):
        seq = [int(rng.integers(K))] * 64
        while len(seq) < 192:
            seq += [int(rng.integers(4))] * int(rng.integers(1, 25))
        seq = seq[:192] + [int(i) for i in rng.integers(K, size=S - 192)]
        idx[:, h] = seq
    qidx = rng.integers(K, size=(S, H))
    qidx[::3] = idx[::3]                      # often read the row just written
    t_, h_ = np.arange(S)[:, None], np.arange(H)[None, :]
    k = np.zeros((1, S, H, K), np.float32)
    k[0, t_, h_, idx] = 1.0
    q = np.zeros((1, S, H, K), np.float32)
    q[0, t_, h_, qidx] = 1.0
    from workloads import GdnInputs, round_bf16
    v = round_bf16(rng.standard_normal((1, S, H, V)).astype(np.float32))
    h0 = (rng.standard_normal((1, H, K, V)) * 0.5).astype(np.float32)
    x = GdnInputs(q, k, v, np.zeros((1, S, H), np.float32), np.ones((1, S, H), np.float32), h0, "bf16", 64,
                  real_tokens=S, name="overwrite-128")
    # the table itself: row idx[t] := v[t], o[t] = row qidx[t] after the write
    st = h0[0].astype(np.float64).copy()
    o = np.zeros((S, H, V))
    for t in range(S):
        for h in range(H):
            st[h, idx[t, h]] = v[0, t, h]
            o[t, h] = st[h, qidx[t, h]]
    return x, o[None], st[None]


@pytest.mark.parametrize("R,reuse_wy", [(1, False), (2, False), (1, True), (4, True)])
def test_overwrite_table_full_size_bf16(R, reuse_wy):
    """Repeated unit keys with beta = 1, g = 0 inside chunks at K = V = 128: the
    GPU result equals the overwrite table (and the oracle), on the recomputing
    scan and on the prepared WY factors, with and without segments."""
    x, o_tab, h_tab = _overwrite_inputs()
    o_ref, h_ref = oracle_forward(x)
    assert rel_err(o_ref, o_tab) < 1e-12 and rel_err(h_ref, h_tab) < 1e-12   # the oracle is the table
    o, hT = run_forward(x, n_segments=R, reuse_wy=reuse_wy)
    check(x, o, hT, o_tab, h_tab, what=f"overwrite R={R} wy={reuse_wy}")


def _signed_gates(x, seed=31):
    """Gates outside the method's usual ranges: a run of increasing decay
    (g > 0) inside a chunk, scattered positive g, and scattered negative beta."""
    rng = np.random.default_rng(seed)
    S = x.g.shape[1]
    x.g = x.g.copy()
    x.beta = x.beta.copy()
    x.g[:, 70:90] = 0.03                      # G rises within chunk 1
    x.g[:, 200::11] = 0.02
    neg = rng.random(x.beta.shape) < 0.15
    x.beta[neg] = -0.3 * x.beta[neg]
    x.name += "-signed-gates"
    assert S > 200
    return x


@pytest.mark.parametrize("R,reuse_wy", [(1, False), (3, False), (1, True)])
def test_signed_gates_bf16(R, reuse_wy):
    """g > 0 and beta < 0 on the matrix-core path give the oracle's result, like
    the vector path (the kernels use the signed exponent of each kept entry and
    multiply beta in, instead of taking its logarithm)."""
    x = _signed_gates(workload(1, H=4, S=1024, decay="slow"))
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, n_segments=R, reuse_wy=reuse_wy)
    check(x, o, hT, o_ref, h_ref, what=f"R={R} wy={reuse_wy}")


def test_signed_gates_f32():
    x = _signed_gates(workload(0, S=256, decay="slow"))
    o_ref, h_ref = oracle_forward(x)
    for R, wy in [(1, False), (2, True)]:
        o, hT = run_forward(x, n_segments=R, reuse_wy=wy)
        check(x, o, hT, o_ref, h_ref, what=f"R={R} wy={wy}")


# ---- gdn_forward: the whole forward in one call -----------------------------------------------

@pytest.mark.parametrize("R", [2, 3, 4])
def test_forward_fused_equals_the_chained_entry_points(R):
    """gdn_forward runs the same kernels in the same order as the chained calls
    (GDN_SCAN_HEAD_EMIT_CARRY, gdn_segment_compose, GDN_SCAN_EMIT), so the
    results are bit-identical; and within tolerance of the oracle."""
    x = workload(1, H=4, S=2048 + 40, decay="slow")
    d = device_inputs(x)
    a = gdn.forward_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], n_segments=R)
    c = gdn.forward_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], n_segments=R)
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])
    o_ref, h_ref = oracle_forward(x)
    check(x, a[0].float().cpu().numpy(), a[1].cpu().numpy(), o_ref, h_ref, what=f"gdn_forward R={R}")


@pytest.mark.parametrize("dtype,K,C", [("bf16", 128, 64), ("f32", 32, 16)])
def test_forward_fused_batch_of_two_with_segments(dtype, K, C):
    """Segments of a batch of two sequences in one call (the Python chain only
    takes one sequence), ragged length, in place (h_out aliasing h0)."""
    x = make_inputs(23, 2, 13 * C + 5, 2, K, K, C, dtype, 0.05, "slow", name=f"fused-b2-{dtype}")
    o_ref, h_ref = oracle_forward(x)
    d = device_inputs(x)
    state = d["h0"].clone()
    o, hT = gdn.forward_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=state, chunk_size=C, n_segments=4,
                              h_out=state)
    torch.cuda.synchronize()
    assert hT.data_ptr() == state.data_ptr()
    check(x, o.float().cpu().numpy(), state.cpu().numpy(), o_ref, h_ref, what="B=2 R=4 in place")


def test_forward_fused_packed_pieces_equals_chained():
    """Packed batch cut into pieces: gdn_forward equals forward_packed's three
    launches bit for bit, with and without final states."""
    x = make_packed_inputs(24, 5, 3000, 2, 128, 128, 64, "bf16", h0_std=0.02, decay="slow", median=400,
                           pad_to_chunk=False, name="fused-packed")
    cu = [int(c) for c in x.cu_seqlens]
    d = device_inputs(x)
    a = gdn.forward_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], cu_seqlens=cu, max_piece_chunks=3)
    c = gdn.forward_packed(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, h0=d["h0"], max_piece_chunks=3)
    a2 = gdn.forward_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], cu_seqlens=cu, max_piece_chunks=3,
                           output_final_state=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]) and torch.equal(a2[0], a[0]) and a2[1] is None
    o_ref, h_ref = oracle_forward(x)
    check(x, a[0][0].float().cpu().numpy(), a[1].cpu().numpy(), o_ref, h_ref, what="gdn_forward pieces")
