"""GPU parity of the backward pass (``gdn_backward`` through the C ABI).

The HIP kernels take the chain rule through the chunk equations of the
MaxText PR "Add context parallelism to the Gated Delta Net" (section "Why");
the oracle takes it through the token recurrence (``oracle.backward``), which
is pinned by finite differences.  Every gradient is compared element by
element, normwise, to the forward tolerances: 1e-4 for fp32 inputs and 2e-2
for bf16 inputs (the kernels compute in fp32; bf16 enters through the inputs
and the rounding of dq, dk, dv).  Cases span several chunks, ragged tails,
both built shapes, packed streams with an empty sequence, absent h0 / dhT
the autograd wrapper and grouped key heads (whose dq, dk are the sums over
the value heads that read them: the chain rule through repeating a key head),
and sequences cut into segments or pieces whose state scans run in parallel
from composed boundary states (checked against the oracle and against the
one-chain backward).
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_gdn_amd as gdn
from chunked_gated_delta_gdn_amd import binding as b
from workloads import make_inputs, make_packed_inputs, make_cotangents
from gpu_util import TOL, DEV, say, to_dev, tdt, rel_err

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def oracle_grads(x, do, dhT, h0=True):
    h0a = x.h0 if h0 else None
    if x.cu_seqlens is not None:
        return oracle.backward_packed(x.cu_seqlens, x.q[0], x.k[0], x.v[0], x.g[0], x.beta[0],
                                      h0a, do[0], dhT)
    return oracle.backward(x.q, x.k, x.v, x.g, x.beta, h0a, do, dhT)


def gpu_grads(x, do, dhT, h0=True, **kw):
    dt = tdt(x.dtype)
    cu = None if x.cu_seqlens is None else [int(c) for c in x.cu_seqlens]
    out = gdn.backward(to_dev(x.q, dt), to_dev(x.k, dt), to_dev(x.v, dt), to_dev(x.g),
                       to_dev(x.beta), to_dev(do, dt),
                       h0=to_dev(x.h0) if (h0 and x.h0 is not None) else None,
                       dhT=None if dhT is None else to_dev(dhT), chunk_size=x.C, cu_seqlens=cu, **kw)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in out]


def check(x, do, dhT, h0=True, tag="", **kw):
    say(f"backward {tag}: {x.name} dtype={x.dtype} shape={x.k.shape} C={x.C} {kw}")
    got = gpu_grads(x, do, dhT, h0, **kw)
    ref = oracle_grads(x, do, dhT, h0)
    if x.cu_seqlens is not None:
        got = [g_[0] if i < 5 else g_ for i, g_ in enumerate(got)]
    errs = {n: rel_err(g_, r) for n, g_, r in zip(NAMES, got, ref)}
    say(f"  errors {errs}")
    for n in NAMES:
        assert errs[n] <= TOL[x.dtype], (n, errs[n])
    return got, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,S,H,K,C", [(2, 37, 2, 32, 16), (1, 200, 2, 128, 64), (2, 64, 1, 128, 64)])
def test_backward_batch(dtype, B, S, H, K, C):
    x = make_inputs(31, B, S, H, K, K, C, dtype, h0_std=0.02, name=f"bwd{B}x{S}")
    do, dhT = make_cotangents(32, x)
    check(x, do, dhT)


@pytest.mark.parametrize("decay", ["slow", "none"])
def test_backward_long_memory(decay):
    # slow decay keeps every chunk's state and its gradient alive across the sequence
    x = make_inputs(33, 1, 300, 2, 128, 128, 64, "f32", h0_std=0.5, decay=decay, name=f"bwd-{decay}")
    do, dhT = make_cotangents(34, x)
    check(x, do, dhT)


def test_backward_without_h0_or_dhT():
    x = make_inputs(35, 1, 150, 2, 128, 128, 64, "bf16", h0_std=0.0, name="bwd-zero-state")
    do, _ = make_cotangents(36, x, dhT_std=0.0)
    got, _ = check(x, do, None, h0=False)
    assert np.isfinite(got[5]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_packed(dtype):
    x = make_packed_inputs(37, 4, 520, 2, 128, 128, 64, dtype, h0_std=0.02, median=120,
                           pad_to_chunk=False, name="bwd-packed")
    # an empty sequence in the middle: dl/dh0 of it must be dl/dhT
    cu = [int(c) for c in x.cu_seqlens]
    x.cu_seqlens = np.array(cu[:2] + [cu[1]] + cu[2:], dtype=np.int32)
    x.h0 = np.concatenate([x.h0[:1], np.full_like(x.h0[:1], 0.3), x.h0[1:]])
    x.meta = {}
    do, dhT = make_cotangents(38, x)
    got, ref = check(x, do, dhT)
    np.testing.assert_array_equal(got[5][1], dhT[1])


def test_backward_packed_small_shape_ragged():
    x = make_packed_inputs(39, 3, 90, 3, 32, 32, 16, "f32", h0_std=0.1, median=30,
                           pad_to_chunk=False, name="bwd-packed-small")
    do, dhT = make_cotangents(40, x)
    check(x, do, dhT)


def test_backward_no_tokens_passes_dhT_through():
    x = make_inputs(41, 2, 0, 2, 32, 32, 16, "f32", h0_std=0.1, name="bwd-empty")
    dhT = np.random.default_rng(42).standard_normal((2, 2, 32, 32)).astype(np.float32)
    do = np.zeros(x.v.shape, dtype=np.float32)
    say("backward: S = 0")
    got = gpu_grads(x, do, dhT)
    np.testing.assert_array_equal(got[5], dhT)


def test_autograd_wrapper():
    x = make_inputs(43, 1, 130, 2, 128, 128, 64, "f32", h0_std=0.02, name="bwd-autograd")
    do, dhT = make_cotangents(44, x)
    say("backward: autograd wrapper")
    q, k, v = (to_dev(a).requires_grad_() for a in (x.q, x.k, x.v))
    g, beta, h0 = (to_dev(a).requires_grad_() for a in (x.g, x.beta, x.h0))
    o, hT = gdn.chunk_gated_delta_rule(q, k, v, g, beta, h0, chunk_size=64)
    loss = (o * to_dev(do)).sum() + (hT * to_dev(dhT)).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle_grads(x, do, dhT)
    for n, t, r in zip(NAMES, (q, k, v, g, beta, h0), ref):
        e = rel_err(t.grad.cpu().numpy(), r)
        assert e <= TOL["f32"], (n, e)


@pytest.mark.parametrize("dtype,H,Hk,packed", [("f32", 4, 2, False), ("bf16", 4, 1, False),
                                              ("f32", 6, 3, True)])
def test_backward_grouped_key_heads(dtype, H, Hk, packed):
    if packed:
        x = make_packed_inputs(45, 3, 260, H, 128, 128, 64, dtype, h0_std=0.02, median=80,
                               pad_to_chunk=False, name="bwd-grouped-packed")
        x.meta = {}
    else:
        x = make_inputs(45, 2, 150, H, 128, 128, 64, dtype, h0_std=0.02, name="bwd-grouped")
    do, dhT = make_cotangents(46, x)
    G = H // Hk
    qg = np.ascontiguousarray(x.q[:, :, ::G])      # key head j = the head that value heads jG .. jG+G-1 read
    kg = np.ascontiguousarray(x.k[:, :, ::G])
    xe = copy.copy(x)
    xe.q, xe.k = oracle.expand_key_heads(qg, H), oracle.expand_key_heads(kg, H)
    say(f"backward grouped {dtype} H={H} Hk={Hk} packed={packed}")
    ref = list(oracle_grads(xe, do, dhT))
    for i in (0, 1):   # repeat -> sum over the group
        r = ref[i]
        ref[i] = r.reshape(r.shape[:-2] + (Hk, G, r.shape[-1])).sum(-2)
    xg = copy.copy(x)
    xg.q, xg.k = qg, kg
    got = gpu_grads(xg, do, dhT)
    if packed:
        got = [g_[0] if i < 5 else g_ for i, g_ in enumerate(got)]
    errs = {n: rel_err(g_, r) for n, g_, r in zip(NAMES, got, ref)}
    say(f"  errors {errs}")
    for n in NAMES:
        assert errs[n] <= TOL[dtype], (n, errs[n])


@pytest.mark.parametrize("wl,heads,R", [(1, (0, 9), 1), (2, (21,), 1), (2, (5,), 4)])
def test_backward_bench_workloads_sampled_heads(wl, heads, R):
    """The backward lines of the benchmark as it times them (4k tokens x 16 heads;
    64k tokens x 32 heads; the latter also cut into 4 segments), every head on
    the GPU, sampled heads through the oracle (heads are independent chains)."""
    from workloads import workload
    x = workload(wl)
    do, dhT = make_cotangents(47, x)
    say(f"backward workload {wl}: {x.k.shape}, R={R}, oracle on heads {heads}")
    got = gpu_grads(x, do, dhT, n_segments=R)
    hs = list(heads)
    ref = oracle.backward(x.q[:, :, hs], x.k[:, :, hs], x.v[:, :, hs], x.g[:, :, hs], x.beta[:, :, hs],
                          x.h0[:, hs], do[:, :, hs], dhT[:, hs])
    for n, g_, r in zip(NAMES, got, ref):
        e = rel_err(g_[:, hs] if n == "dh0" else g_[:, :, hs], r)
        say(f"  {n}: {e:.3e}")
        assert e <= TOL[x.dtype], (n, e)


def test_backward_is_deterministic():
    """Two calls on the same inputs give the same bits: every reduction (dg and
    dbeta included) runs in a fixed order, none through floating-point atomics."""
    x = make_inputs(48, 1, 1000, 4, 128, 128, 64, "bf16", h0_std=0.02, decay="slow", name="bwd-det")
    do, dhT = make_cotangents(49, x)
    say("backward: determinism")
    for kw in ({}, {"n_segments": 3}):
        a = gpu_grads(x, do, dhT, **kw)
        b = gpu_grads(x, do, dhT, **kw)
        for n, u, v in zip(NAMES, a, b):
            np.testing.assert_array_equal(u, v, err_msg=f"{n} {kw}")


def _vs_one_chain(x, got, whole):
    """Cut chains against the one-chain backward: fp32 outputs agree to 1e-5
    normwise (only the rounding of the composed maps differs); outputs stored in
    bf16 (dq, dk, dv of bf16 inputs) to two units in the last place."""
    worst = 0.0
    for i, (n, u, w) in enumerate(zip(NAMES, got, whole)):
        e = rel_err(u, w)
        tol = 8e-3 if (x.dtype == "bf16" and i < 3) else 1e-5
        say(f"  {n} vs one chain: {e:.3e} (bound {tol:g})")
        assert e <= tol, (n, e)
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("dtype,B,R,seg_starts", [("f32", 2, 2, None), ("f32", 1, 4, None),
                                                  ("bf16", 1, 4, [0, 64, 320, 448]), ("bf16", 2, 2, None)])
def test_backward_segments(dtype, B, R, seg_starts):
    """Segments cut each sequence's two state scans into parts scanned at once:
    the state scan's carries (M, U) compose the parts' start states, the reverse
    scan's (M^T, E) their end gradients.  Slow decay keeps the state and its
    gradient alive across every boundary, so a wrong carry or compose shows."""
    x = make_inputs(53, B, 600, 2, 128, 128, 64, dtype, h0_std=0.3, decay="slow", name=f"bwd-seg{R}")
    do, dhT = make_cotangents(54, x)
    got, _ = check(x, do, dhT, tag=f"R={R}", n_segments=R, seg_starts=seg_starts)
    _vs_one_chain(x, got, gpu_grads(x, do, dhT))


def test_backward_segments_small_shape():
    x = make_inputs(55, 2, 150, 3, 32, 32, 16, "f32", h0_std=0.3, decay="slow", name="bwd-seg-small")
    do, dhT = make_cotangents(56, x)
    got, _ = check(x, do, dhT, tag="R=3", n_segments=3)
    _vs_one_chain(x, got, gpu_grads(x, do, dhT))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_pieces(dtype):
    """A packed batch cut into pieces of at most 2 chunks (an empty sequence
    and a one-piece sequence among them): oracle parity and agreement with the
    one-chain backward."""
    x = make_packed_inputs(57, 4, 900, 2, 128, 128, 64, dtype, h0_std=0.3, median=250, decay="slow",
                           pad_to_chunk=False, name="bwd-pieces")
    cu = [int(c) for c in x.cu_seqlens]
    x.cu_seqlens = np.array(cu[:2] + [cu[1]] + cu[2:], dtype=np.int32)
    x.h0 = np.concatenate([x.h0[:1], np.full_like(x.h0[:1], 0.3), x.h0[1:]])
    x.meta = {}
    do, dhT = make_cotangents(58, x)
    p = gdn.problem_for(to_dev(x.k, tdt(dtype)), to_dev(x.v, tdt(dtype)), 64,
                        [int(c) for c in x.cu_seqlens], max_piece_chunks=2)
    assert b.gdn_num_pieces(p) > len(x.cu_seqlens) + 1
    got, _ = check(x, do, dhT, tag="pieces", max_piece_chunks=2)
    np.testing.assert_array_equal(got[5][1], dhT[1])
    whole = gpu_grads(x, do, dhT)
    whole = [g_[0] if i < 5 else g_ for i, g_ in enumerate(whole)]
    _vs_one_chain(x, got, whole)


@pytest.mark.parametrize("mode", ["segments", "packed_pieces"])
def test_autograd_wrapper_with_forward_schedules(mode):
    """The differentiable forward with segments or a packed batch cut into pieces:
    the schedule changes the launches (the backward's state scans take the same
    cut), not the result: the oracle's gradients."""
    if mode == "segments":
        x = make_inputs(50, 1, 700, 2, 128, 128, 64, "bf16", h0_std=0.02, decay="slow", name="bwd-seg")
        kw = dict(n_segments=3)
    else:
        x = make_packed_inputs(51, 3, 900, 2, 128, 128, 64, "bf16", h0_std=0.02, median=300,
                               pad_to_chunk=False, name="bwd-pieces")
        x.meta = {}
        kw = dict(cu_seqlens=[int(c) for c in x.cu_seqlens], max_piece_chunks=2)
        # the forward really is cut into pieces (sequences of 4, 4 and 7 chunks)
        p = gdn.problem_for(to_dev(x.k, torch.bfloat16), to_dev(x.v, torch.bfloat16), 64, kw["cu_seqlens"],
                            max_piece_chunks=2)
        assert b.gdn_num_pieces(p) > len(x.cu_seqlens) - 1
    do, dhT = make_cotangents(52, x)
    say(f"backward: autograd with {mode}")
    bf = torch.bfloat16
    q, k, v = (to_dev(a, bf).requires_grad_() for a in (x.q, x.k, x.v))
    g, beta, h0 = (to_dev(a).requires_grad_() for a in (x.g, x.beta, x.h0))
    o, hT = gdn.chunk_gated_delta_rule(q, k, v, g, beta, h0, chunk_size=64, **kw)
    loss = (o.float() * to_dev(do)).sum() + (hT * to_dev(dhT)).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle_grads(x, do, dhT)
    for n, t, r in zip(NAMES, (q, k, v, g, beta, h0), ref):
        gr = t.grad.float().cpu().numpy()
        if x.cu_seqlens is not None and n != "dh0":
            gr = gr[0]
        e = rel_err(gr, r)
        say(f"  {n}: {e:.3e}")
        assert e <= TOL["bf16"], (n, e)
