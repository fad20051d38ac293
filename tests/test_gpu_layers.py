"""GPU parity of the steps beside the core -- the depthwise causal conv with its
state, and the gated RMSNorm -- against the fp64 oracle (``oracle/layers.py``),
through the C ABI.  Bounds: normwise relative error <= 1e-5 for fp32 (the
arithmetic is a handful of fp32 operations per value) and <= 1e-2 for bf16
(one bf16 rounding of the result, 2^-9, with margin)."""
import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_gdn_amd as gdn
from workloads import round_bf16
from gpu_util import DEV, say, rel_err, to_dev

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


def vals(rng, shape, dtype, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def tdt(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def conv_case(seed, T, D, W, dtype, N, with_state):
    rng = np.random.default_rng(seed)
    x = vals(rng, (T, D), dtype)
    w = vals(rng, (D, W), dtype, 0.5)
    st = vals(rng, (N, D, W - 1), dtype) if with_state else None
    return x, w, st


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("with_state", [False, True])
def test_conv_batch(dtype, W, with_state):
    B, S, D = 2, 150, 300          # D not a multiple of the 256-channel workgroup
    rng = np.random.default_rng(W)
    x = vals(rng, (B, S, D), dtype)
    w = vals(rng, (D, W), dtype, 0.5)
    st = vals(rng, (B, D, W - 1), dtype) if with_state else None
    for act in ("none", "silu"):
        y, s2 = gdn.causal_conv1d(to_dev(x, tdt(dtype)), to_dev(w, tdt(dtype)),
                                  None if st is None else to_dev(st, tdt(dtype)), activation=act)
        torch.cuda.synchronize()
        for b in range(B):
            y_ref, s_ref = oracle.causal_conv1d(x[b], w, None if st is None else st[b], activation=act)
            ey = rel_err(y[b].float().cpu().numpy(), y_ref)
            say(f"  conv batch {dtype} W={W} state={with_state} {act} b={b}: err(y)={ey:.2e}")
            assert ey <= TOL[dtype]
            # the new state is made of input values: exact
            np.testing.assert_array_equal(s2[b].float().cpu().numpy(), s_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
def test_conv_eight_channel_runs(dtype, W):
    """Channel counts that are a multiple of 8 take the streaming 8-channel
    kernels (bf16 with at most 4 taps: the bf16 dot-product kernel): every tap
    count, a ragged last run (150 = 2 x 64 + 22 tokens), a partial channel
    group (264 channels), with and without a state, both activations."""
    B, S, D = 2, 150, 264
    rng = np.random.default_rng(100 + W)
    x = vals(rng, (B, S, D), dtype)
    w = vals(rng, (D, W), dtype, 0.5)
    for with_state in (False, True):
        st = vals(rng, (B, D, W - 1), dtype) if with_state else None
        for act in ("none", "silu"):
            y, s2 = gdn.causal_conv1d(to_dev(x, tdt(dtype)), to_dev(w, tdt(dtype)),
                                      None if st is None else to_dev(st, tdt(dtype)), activation=act)
            torch.cuda.synchronize()
            for b in range(B):
                y_ref, s_ref = oracle.causal_conv1d(x[b], w, None if st is None else st[b], activation=act)
                ey = rel_err(y[b].float().cpu().numpy(), y_ref)
                say(f"  conv 8-channel {dtype} W={W} state={with_state} {act} b={b}: err(y)={ey:.2e}")
                assert ey <= TOL[dtype]
                np.testing.assert_array_equal(s2[b].float().cpu().numpy(), s_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 3])
def test_conv_packed_short_sequences_few_taps(dtype, W):
    """Packed sequences shorter than the window with 2 or 3 taps on the
    8-channel kernels: the positions before a sequence come from its state
    (W - 1 of them) and the padded taps see zeros beyond it."""
    lens = [1, 2, 3, 0, 5, 66]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, D = int(cu[-1]), 136
    x, w, st = conv_case(7 + W, T, D, W, dtype, len(lens), True)
    y, s2 = gdn.causal_conv1d(to_dev(x[None], tdt(dtype)), to_dev(w, tdt(dtype)), to_dev(st, tdt(dtype)),
                              cu_seqlens=cu)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.causal_conv1d_packed(x, w, cu, st)
    ey = rel_err(y[0].float().cpu().numpy(), y_ref)
    say(f"  conv packed short {dtype} W={W}: err(y)={ey:.2e}")
    assert ey <= TOL[dtype]
    np.testing.assert_array_equal(s2.float().cpu().numpy(), s_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_packed_ragged_empty_and_short(dtype):
    """Packed sequences of lengths 0, 1, 2, 63, 64, 65, 130 (some crossing
    64-token block boundaries, some shorter than the state)."""
    lens = [70, 0, 1, 2, 63, 0, 64, 65, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, D, W = int(cu[-1]), 520, 4
    x, w, st = conv_case(5, T, D, W, dtype, len(lens), True)
    y, s2 = gdn.causal_conv1d(to_dev(x[None], tdt(dtype)), to_dev(w, tdt(dtype)), to_dev(st, tdt(dtype)),
                              cu_seqlens=cu)
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.causal_conv1d_packed(x, w, cu, st)
    ey = rel_err(y[0].float().cpu().numpy(), y_ref)
    say(f"  conv packed {dtype}: err(y)={ey:.2e}")
    assert ey <= TOL[dtype]
    np.testing.assert_array_equal(s2.float().cpu().numpy(), s_ref)
    # empty sequences keep their state
    np.testing.assert_array_equal(s2[1].float().cpu().numpy(), st[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_decode_steps_in_place_equal_one_pass(dtype):
    """Decode: 6 one-token steps of 5 sequences, the state updated in place,
    reproduce the convolution of the 6 tokens in one pass (GPU against GPU and
    against the oracle)."""
    N, D, W, steps = 5, 256, 4, 6
    rng = np.random.default_rng(6)
    x = vals(rng, (steps, N, D), dtype)
    w = vals(rng, (D, W), dtype, 0.5)
    st0 = vals(rng, (N, D, W - 1), dtype)
    state = to_dev(st0, tdt(dtype))
    ys = []
    for s in range(steps):
        y, _ = gdn.causal_conv1d(to_dev(x[s][:, None], tdt(dtype)), to_dev(w, tdt(dtype)), state, state_out=state)
        ys.append(y[:, 0])
    torch.cuda.synchronize()
    seq = np.ascontiguousarray(x.transpose(1, 0, 2))           # [N, steps, D]
    y1, s1 = gdn.causal_conv1d(to_dev(seq, tdt(dtype)), to_dev(w, tdt(dtype)), to_dev(st0, tdt(dtype)))
    torch.cuda.synchronize()
    yd = torch.stack(ys, 1)
    assert torch.equal(yd, y1) and torch.equal(state, s1)
    for n in range(N):
        y_ref, s_ref = oracle.causal_conv1d(seq[n], w, st0[n])
        assert rel_err(yd[n].float().cpu().numpy(), y_ref) <= TOL[dtype]
        np.testing.assert_array_equal(state[n].float().cpu().numpy(), s_ref)


def test_conv_state_alias_rule():
    """In-place state across a sequence that spans two token blocks is refused
    (it would race); one-token sequences may update in place."""
    D, W = 64, 4
    x = torch.zeros((1, 130, D), device=DEV)
    w = torch.zeros((D, W), device=DEV)
    st = torch.zeros((1, D, W - 1), device=DEV)
    with pytest.raises(ValueError, match="alias"):
        gdn.causal_conv1d(x, w, st, state_out=st)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [32, 128, 200])
@pytest.mark.parametrize("gated", [False, True])
def test_gated_rmsnorm(dtype, V, gated):
    rng = np.random.default_rng(V)
    rows = 777
    o = vals(rng, (rows, V), dtype, 3.0)
    z = vals(rng, (rows, V), dtype) if gated else None
    w = rng.standard_normal(V).astype(np.float32)
    y = gdn.gated_rmsnorm(to_dev(o, tdt(dtype)), to_dev(w), None if z is None else to_dev(z, tdt(dtype)), eps=1e-6)
    torch.cuda.synchronize()
    y_ref = oracle.gated_rmsnorm(o, w, z, eps=1e-6)
    e = rel_err(y.float().cpu().numpy(), y_ref)
    say(f"  gated rmsnorm {dtype} V={V} gated={gated}: err={e:.2e}")
    assert e <= TOL[dtype]


def test_gated_rmsnorm_in_place_and_zero_rows():
    rng = np.random.default_rng(9)
    o = rng.standard_normal((3, 5, 128)).astype(np.float32)
    o[1, 2] = 0.0                                             # a zero row stays zero (eps > 0)
    w = rng.standard_normal(128).astype(np.float32)
    t = to_dev(o)
    y = gdn.gated_rmsnorm(t, to_dev(w), eps=1e-6, out=t)
    torch.cuda.synchronize()
    assert y.data_ptr() == t.data_ptr()
    assert rel_err(y.cpu().numpy(), oracle.gated_rmsnorm(o, w, eps=1e-6)) <= TOL["f32"]
    assert not np.any(y[1, 2].cpu().numpy())


def test_conv_and_norm_bench_size_sampled():
    """The conv and the norm at the sizes the benchmark times them (65,536 tokens;
    conv over 8,192 channels, 4 taps, SiLU, with a state; norm over 32 heads of
    128 values with a gate, bf16), in that launch configuration: every output on the
    GPU, sampled channels (conv: 64 channels from each 2,048-channel workgroup
    column) and rows (norm: 4,096 rows) through the oracle."""
    Tn, D, W, H, V = 65536, 8192, 4, 32, 128
    rng = np.random.default_rng(61)
    x = round_bf16(rng.standard_normal((1, Tn, D), dtype=np.float32))
    w = vals(rng, (D, W), "bf16", 0.5)
    st = vals(rng, (1, D, W - 1), "bf16")
    say(f"conv at bench size: T={Tn} D={D} W={W}")
    y, s2 = gdn.causal_conv1d(to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16), to_dev(st, torch.bfloat16))
    torch.cuda.synchronize()
    ch = np.concatenate([np.arange(64) + 2048 * c for c in range(4)]) + 7
    ch = ch[ch < D]
    y_ref, s_ref = oracle.causal_conv1d(x[0][:, ch], w[ch], st[0][ch])
    ey = rel_err(y[0][:, ch].float().cpu().numpy(), y_ref)
    say(f"  conv sampled channels: err(y)={ey:.2e}")
    assert ey <= TOL["bf16"]
    np.testing.assert_array_equal(s2[0][ch].float().cpu().numpy(), s_ref)
    del x, y, s2
    o = round_bf16(rng.standard_normal((Tn, H, V), dtype=np.float32) * 3.0)
    z = round_bf16(rng.standard_normal((Tn, H, V), dtype=np.float32))
    wn = rng.standard_normal(V).astype(np.float32)
    say(f"norm at bench size: rows={Tn * H} V={V}")
    yn = gdn.gated_rmsnorm(to_dev(o, torch.bfloat16), to_dev(wn), to_dev(z, torch.bfloat16))
    torch.cuda.synchronize()
    rows = rng.choice(Tn, size=128, replace=False)
    yr = oracle.gated_rmsnorm(o[rows].reshape(-1, V), wn, z[rows].reshape(-1, V))
    e = rel_err(yn[torch.as_tensor(rows, device=yn.device)].float().cpu().numpy().reshape(-1, V), yr)
    say(f"  norm sampled rows: err={e:.2e}")
    assert e <= TOL["bf16"]
