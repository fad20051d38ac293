"""GPU parity of packed batches cut into pieces (the segment pass run per
sequence of a packed batch, so that a long sequence becomes parallel chains)
against the fp64 oracle, through the C ABI.  Bounds as everywhere: normwise
relative error <= 1e-4 (fp32 inputs) and <= 2e-2 (bf16 inputs) on the outputs
and the final states.  Slow decay keeps the carried M of every piece alive, so
a wrong M, a wrong piece boundary or a wrong state row would show."""
import numpy as np
import pytest
import torch

import chunked_gated_delta_gdn_amd as gdn
from workloads import make_inputs, workload
from gpu_util import TOL, DEV, say, device_inputs, oracle_forward, rel_err, run_forward, check_forward

pytestmark = pytest.mark.gpu


def packed(seed, cu, H, K, C, dtype, decay="slow", h0_std=0.1):
    rng = np.random.default_rng(seed)
    x = make_inputs(seed, 1, int(cu[-1]), H, K, K, C, dtype, 0.0, decay, name=f"pieces{seed}")
    x.cu_seqlens = np.asarray(cu, dtype=np.int32)
    x.h0 = rng.standard_normal((len(cu) - 1, H, K, K)).astype(np.float32) * h0_std
    return x


def check(x, o, hT, o_ref, h_ref, what):
    check_forward(x, o, hT, o_ref, h_ref, what=what)


# chunks per sequence at C = 16: 3, 0, 8, 1, 28 (ragged tails, an empty and a one-token sequence)
CU16 = [0, 37, 37, 160, 161, 600]


@pytest.mark.parametrize("m", [1, 2, 3, 8])
@pytest.mark.parametrize("schedule", ["auto", "plain"])
def test_pieces_f32(m, schedule):
    x = packed(31, CU16, 2, 32, 16, "f32")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, schedule=schedule, max_piece_chunks=m)
    check(x, o[0], hT, o_ref, h_ref, f"m={m} {schedule}")
    np.testing.assert_array_equal(hT[1], x.h0[1])   # the empty sequence keeps its state


@pytest.mark.parametrize("m", [1, 3])
def test_pieces_f32_reuse_wy(m):
    x = packed(32, CU16, 2, 32, 16, "f32")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, reuse_wy=True, max_piece_chunks=m)
    check(x, o[0], hT, o_ref, h_ref, f"m={m} wy reused")


# chunks per sequence at C = 64: 16, 0, 3, 10 (ragged last one)
CU64 = [0, 1000, 1000, 1130, 1767]


@pytest.mark.parametrize("m", [1, 2, 5, 16])
@pytest.mark.parametrize("schedule", ["auto", "plain"])
def test_pieces_bf16_128(m, schedule):
    x = packed(33, CU64, 2, 128, 64, "bf16", h0_std=0.02)
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, schedule=schedule, max_piece_chunks=m)
    check(x, o[0], hT, o_ref, h_ref, f"m={m} {schedule}")
    np.testing.assert_array_equal(hT[1], x.h0[1])


@pytest.mark.parametrize("m", [1, 4])
def test_pieces_bf16_128_reuse_wy(m):
    x = packed(34, CU64, 2, 128, 64, "bf16", h0_std=0.02)
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, reuse_wy=True, max_piece_chunks=m)
    check(x, o[0], hT, o_ref, h_ref, f"m={m} wy reused")


def test_pieces_match_whole_sequences_config_decay():
    """The configuration decay (mean alpha about 0.5): pieces against the
    whole-sequence scan on the GPU and against the oracle."""
    x = packed(35, CU64, 3, 128, 64, "bf16", decay="config", h0_std=0.02)
    o_ref, h_ref = oracle_forward(x)
    o1, h1 = run_forward(x, max_piece_chunks=0)
    o2, h2 = run_forward(x, max_piece_chunks=3)
    check(x, o2[0], h2, o_ref, h_ref, "m=3")
    assert rel_err(o2, o1) <= TOL["bf16"] and rel_err(h2, h1) <= TOL["bf16"]


def test_head_and_tail_calls_compose_to_the_plain_pass():
    """The three calls of forward_packed one by one: the first pieces' outputs
    and states come from the head call alone; the tail call leaves them alone."""
    x = packed(36, CU16, 2, 32, 16, "f32")
    d = device_inputs(x)
    cu, m = x.cu_seqlens, 3
    o = torch.full(d["v"].shape, 5.0, device=DEV)
    N = len(cu) - 1
    hT = torch.full((N, 2, 32, 32), 9.0, device=DEV)
    _, _, M, U = gdn.scan_head_carry(d["q"], d["k"], d["v"], d["g"], d["beta"], h_in=d["h0"], chunk_size=16,
                                     out=o, cu_seqlens=cu, max_piece_chunks=m, h_out=hT)
    h1 = hT.clone()
    o_head = o.clone()
    h_in, _ = gdn.piece_compose(d["k"], d["v"], M, U, cu, m, 16, first=1, h_seed=h1)
    gdn.scan_tail_emit(d["q"], d["k"], d["v"], d["g"], d["beta"], h_in, cu, m, chunk_size=16, out=o, h_out=hT)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_forward(x)
    check(x, o[0].cpu().numpy(), hT.cpu().numpy(), o_ref, h_ref, "head, compose, tail")
    # first piece of each sequence: ceil-free split rule, piece 0 has c * 1 // R chunks
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        nc = -(-(b - a) // 16)
        R = -(-nc // m) if nc > m else 1
        end = min(b, a + 16 * (nc // R)) if R > 1 else b
        assert torch.equal(o[0, a:end], o_head[0, a:end])          # tail did not touch them
        if R > 1:
            assert bool((o_head[0, end:b] == 5.0).all())          # head did not write the rest
        else:
            assert torch.equal(hT[n], h1[n])                       # one-piece sequences keep head's state


def test_packed_config_plans_pieces_and_matches_oracle():
    """The packed 8-sequence, 32k-token, 32-head workload: the planner cuts its
    longest sequence (20,623 tokens) into pieces; three sampled heads are
    recomputed by the oracle in full."""
    x = workload(3)
    chunks = tuple(-(-(int(x.cu_seqlens[n + 1]) - int(x.cu_seqlens[n])) // 64) for n in range(8))
    n_cu = torch.cuda.get_device_properties(DEV).multi_processor_count
    m = gdn.plan_pieces(chunks, 32, n_cu)
    assert m > 0
    o, hT = run_forward(x)
    heads = [0, 13, 30]
    o_ref, h_ref = oracle_forward(x, heads=heads)
    check(x, o[0][:, heads], hT[:, heads], o_ref, h_ref, f"planned m={m}, heads {heads}")


@pytest.mark.parametrize("m", ["auto", 2])
def test_batch_given_pieces_runs_as_packed(m):
    """A [B,S,H,*] batch with max_piece_chunks runs as the packed batch of its
    B sequences: same results as the oracle per sequence."""
    x = make_inputs(37, 2, 300, 2, 32, 32, 16, "f32", 0.1, "slow", name="batch-pieces")
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x, max_piece_chunks=m)
    assert o.shape == (2, 300, 2, 32)
    check(x, o, hT, o_ref, h_ref, f"batch m={m}")


@pytest.mark.parametrize("dtype,K,C", [("f32", 32, 16), ("bf16", 128, 64)])
def test_mixed_prefill_and_decode_batch(dtype, K, C):
    """A packed batch mixing prefills and one-token decode requests, each
    request with its own state: the decode requests' outputs and states equal
    gdn_decode_step on the same token and state (to the tolerance: the chunked
    and the single-token kernels round differently), and every sequence follows
    the oracle."""
    lens = [5 * C + 3, 1, 2 * C, 1, 1, 3 * C + 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = packed(45, cu, 2, K, C, dtype, h0_std=0.05)
    o_ref, h_ref = oracle_forward(x)
    o, hT = run_forward(x)
    check(x, o[0], hT, o_ref, h_ref, "mixed prefill/decode")
    d = device_inputs(x)
    dt = d["k"].dtype
    for n, L in enumerate(lens):
        if L != 1:
            continue
        t = int(cu[n])
        state = d["h0"][n:n + 1].clone()
        tok = {n_: d[n_][0, t:t + 1].clone() for n_ in ("q", "k", "v", "g", "beta")}   # aligned copies
        od = gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], state)
        torch.cuda.synchronize()
        assert rel_err(o[0, t], od[0].float().cpu().numpy()) <= TOL[dtype]
        assert rel_err(hT[n], state[0].cpu().numpy()) <= TOL[dtype]
