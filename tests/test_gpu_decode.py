"""GPU parity of the recurrent decode step against the fp64 oracle (through
the C ABI), and its consistency with the chunked forward."""
import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_gdn_amd as gdn
from workloads import make_decode_inputs, make_inputs
from gpu_util import TOL, say, rel_err, tdt, to_dev, oracle_forward, run_forward

pytestmark = pytest.mark.gpu


def _run_steps(d, steps, keep=()):
    dt = tdt(d.dtype)
    state = to_dev(d.state0)
    outs, kept = [], {}
    for t in range(steps):
        o = gdn.decode_step(to_dev(d.q[t], dt), to_dev(d.k[t], dt), to_dev(d.v[t], dt),
                            to_dev(d.g[t]), to_dev(d.beta[t]), state)
        outs.append(o.float().cpu().numpy())
        if t + 1 in keep:
            kept[t + 1] = state.cpu().numpy()
    torch.cuda.synchronize()
    return np.stack(outs), state.cpu().numpy(), kept


@pytest.mark.parametrize("dtype,K", [("f32", 32), ("bf16", 32), ("f32", 128), ("bf16", 128)])
def test_decode_small(dtype, K):
    d = make_decode_inputs(40 + K, 3, 4, K, K, 5, dtype=dtype)
    o, st, _ = _run_steps(d, 5)
    state = d.state0.astype(np.float64)
    for t in range(5):
        o_ref, state = oracle.decode_step(d.q[t], d.k[t], d.v[t], d.g[t], d.beta[t], state)
        e = rel_err(o[t], o_ref)
        assert e <= TOL[dtype], (t, e)
    assert rel_err(st, state) <= TOL[dtype]


def test_decode_b256_h32_128_steps_sampled():
    """The batched decode workload (B256 H32 K=V=128, fp32 state 512 MiB, 128
    steps); the oracle follows 24 sampled (b, h) chains through all steps."""
    steps = 128
    d = make_decode_inputs(4, 256, 32, 128, 128, steps, dtype="bf16")
    o, st, kept = _run_steps(d, steps, keep=(1,))
    rng = np.random.default_rng(0)
    bs = rng.choice(256, 24, replace=False)
    hs = rng.integers(0, 32, size=24)
    state = d.state0[bs, hs].astype(np.float64)[:, None]          # [24,1,K,V]
    worst = 0.0
    for t in range(steps):
        o_ref, state = oracle.decode_step(d.q[t][bs, hs][:, None], d.k[t][bs, hs][:, None],
                                          d.v[t][bs, hs][:, None], d.g[t][bs, hs][:, None],
                                          d.beta[t][bs, hs][:, None], state)
        worst = max(worst, rel_err(o[t][bs, hs], o_ref[:, 0]))
        if t == 0:
            assert rel_err(kept[1][bs, hs], state[:, 0]) <= TOL["bf16"]
    say(f"  decode B256 H32: worst err(o) over 128 steps {worst:.3e}, "
        f"err(state) {rel_err(st[bs, hs], state[:, 0]):.3e}")
    assert worst <= TOL["bf16"]
    assert rel_err(st[bs, hs], state[:, 0]) <= TOL["bf16"]


def test_decode_steps_equal_chunked_forward():
    """128 decode steps == one chunked forward over the same 128 tokens."""
    d = make_decode_inputs(9, 2, 4, 128, 128, 128, dtype="bf16")
    o, st, _ = _run_steps(d, 128)
    sw = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))
    x = make_inputs(0, 2, 128, 4, 128, 128, 64, "bf16")
    x.q, x.k, x.v, x.g, x.beta, x.h0 = sw(d.q), sw(d.k), sw(d.v), sw(d.g), sw(d.beta), d.state0
    o_f, h_f = run_forward(x)
    assert rel_err(sw(o), o_f) <= TOL["bf16"]
    assert rel_err(st, h_f) <= TOL["bf16"]
