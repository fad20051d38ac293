"""GPU parity with grouped key heads: q and k have H_qk heads for H value heads,
value head h reading key head h // (H / H_qk) ("RFC(qwen35): TP Phase 2",
section "Partition Contract"; grouped order as on the Ulysses page).  The
oracle runs the ungrouped definition on q, k with each key head repeated in
place; the GPU's grouped run must also equal its own run on those repeated
inputs bit for bit (same values through the same kernels)."""
import copy

import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_gdn_amd as gdn
from workloads import make_inputs, make_decode_inputs
from gpu_util import TOL, DEV, say, oracle_forward, rel_err, run_forward, to_dev, check_forward

pytestmark = pytest.mark.gpu


def grouped(seed, B, S, H, Hk, K, C, dtype, h0_std, decay):
    """Seeded inputs with H value heads, keeping key heads 0 .. Hk-1 of q and k."""
    x = make_inputs(seed, B, S, H, K, K, C, dtype, h0_std, decay, name=f"grouped{H}/{Hk}")
    x.q = np.ascontiguousarray(x.q[:, :, :Hk])
    x.k = np.ascontiguousarray(x.k[:, :, :Hk])
    return x


def expanded(x):
    """The same problem with each key head repeated in grouped order."""
    y = copy.copy(x)
    H = x.v.shape[2]
    y.q = np.ascontiguousarray(oracle.expand_key_heads(x.q, H))
    y.k = np.ascontiguousarray(oracle.expand_key_heads(x.k, H))
    return y


def check(x, o, hT, o_ref, h_ref, what):
    check_forward(x, o, hT, o_ref, h_ref, what=what)


@pytest.mark.parametrize("Hk", [1, 2])
@pytest.mark.parametrize("R", [1, 3])
def test_grouped_f32(Hk, R):
    x = grouped(41, 1, 300, 4, Hk, 32, 16, "f32", 0.1, "slow")
    o_ref, h_ref = oracle_forward(expanded(x))
    o, hT = run_forward(x, n_segments=R)
    check(x, o, hT, o_ref, h_ref, f"R={R}")
    oe, he = run_forward(expanded(x), n_segments=R)
    assert np.array_equal(o, oe) and np.array_equal(hT, he)


@pytest.mark.parametrize("R,wy", [(1, False), (4, False), (2, True)])
def test_grouped_bf16_128(R, wy):
    x = grouped(42, 1, 700, 4, 2, 128, 64, "bf16", 0.02, "slow")
    o_ref, h_ref = oracle_forward(expanded(x))
    o, hT = run_forward(x, n_segments=R, reuse_wy=wy)
    check(x, o, hT, o_ref, h_ref, f"R={R} wy={wy}")
    oe, he = run_forward(expanded(x), n_segments=R, reuse_wy=wy)
    assert np.array_equal(o, oe) and np.array_equal(hT, he)


@pytest.mark.parametrize("dtype,K,C", [("f32", 32, 16), ("bf16", 128, 64)])
def test_grouped_packed_pieces(dtype, K, C):
    cu = np.array([0, 9 * C + 5, 9 * C + 5, 12 * C], dtype=np.int32)
    x = grouped(43, 1, int(cu[-1]), 4, 2, K, C, dtype, 0.0, "slow")
    x.cu_seqlens = cu
    x.h0 = np.random.default_rng(43).standard_normal((3, 4, K, K)).astype(np.float32) * 0.05
    o_ref, h_ref = oracle_forward(expanded(x))
    o, hT = run_forward(x, max_piece_chunks=2)
    check(x, o[0], hT, o_ref, h_ref, "packed, pieces of 2 chunks")


@pytest.mark.parametrize("dtype,K", [("f32", 32), ("bf16", 128)])
def test_grouped_decode(dtype, K):
    d = make_decode_inputs(44, 8, 4, K, K, 3, dtype=dtype)
    Hk = 2
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k = d.q[:, :, :Hk], d.k[:, :, :Hk]                      # [steps, B, Hk, K]
    state = to_dev(d.state0)
    state_e = to_dev(d.state0)
    ref = d.state0.astype(np.float64)
    for s in range(3):
        o = gdn.decode_step(to_dev(q[s], dt), to_dev(k[s], dt), to_dev(d.v[s], dt), to_dev(d.g[s]),
                            to_dev(d.beta[s]), state)
        qe, ke = oracle.expand_key_heads(q[s], 4), oracle.expand_key_heads(k[s], 4)
        oe = gdn.decode_step(to_dev(qe, dt), to_dev(ke, dt), to_dev(d.v[s], dt), to_dev(d.g[s]),
                             to_dev(d.beta[s]), state_e)
        o_ref, ref = oracle.decode_step(qe, ke, d.v[s], d.g[s], d.beta[s], ref)
        torch.cuda.synchronize()
        eo, es = rel_err(o.float().cpu().numpy(), o_ref), rel_err(state.cpu().numpy(), ref)
        say(f"  grouped decode {dtype} step {s}: err(o)={eo:.3e} err(state)={es:.3e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]
        assert torch.equal(o, oe) and torch.equal(state, state_e)
