"""The entry points captured in HIP graphs (torch.cuda.CUDAGraph on ROCm):
every replay, with eager work and synchronisations between replays, equals the
eager result bit for bit.  Nothing on these paths records a memset node or
synchronises inside the capture."""
import numpy as np
import pytest
import torch

import chunked_gated_delta_gdn_amd as gdn
from workloads import make_decode_inputs, workload
from gpu_util import DEV, device_inputs, to_dev

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def test_segmented_forward_in_a_graph():
    x = workload(1, H=4, decay="slow")
    d = device_inputs(x)
    run = lambda: gdn.forward_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], chunk_size=64,
                                        n_segments=4)
    o_ref, h_ref = run()
    torch.cuda.synchronize()
    g, (o, h) = capture(run)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(h, h_ref)
        o2, h2 = run()                         # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref)


def test_packed_pieces_forward_in_a_graph():
    x = workload(3, H=4)
    d = device_inputs(x)
    cu = x.cu_seqlens
    run = lambda: gdn.forward_packed(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, h0=d["h0"], chunk_size=64,
                                     max_piece_chunks=40)
    o_ref, h_ref = run()
    torch.cuda.synchronize()
    g, (o, h) = capture(run)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(h, h_ref)
        run()
        torch.cuda.synchronize()


def test_decode_steps_in_a_graph():
    """Four decode steps captured once; each replay advances the captured state
    by four tokens, like four eager steps on a copy of it."""
    dd = make_decode_inputs(3, 8, 4, 128, 128, 4, dtype="bf16")
    bf = torch.bfloat16
    q, k, v = to_dev(dd.q, bf), to_dev(dd.k, bf), to_dev(dd.v, bf)
    gg, bb = to_dev(dd.g), to_dev(dd.beta)
    state = to_dev(dd.state0)
    ref_state = state.clone()
    out = torch.empty((4, 8, 4, 128), dtype=bf, device=DEV)
    ref_out = torch.empty_like(out)

    def steps(st, o):
        for s in range(4):
            gdn.decode_step(q[s], k[s], v[s], gg[s], bb[s], st, out=o[s])
        return o
    g, _ = capture(lambda: steps(state, out))
    # the warm-up and capture ran the steps once eagerly: bring the reference along
    steps(ref_state, ref_out)
    torch.cuda.synchronize()
    assert torch.equal(state, ref_state)
    for _ in range(3):
        g.replay()
        steps(ref_state, ref_out)
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state) and torch.equal(out, ref_out)


def test_backward_in_a_graph():
    """gdn_backward (four kernels, grouped key heads: five) captured once; every
    replay reproduces the eager gradients bit for bit."""
    from workloads import make_cotangents
    for Hk in (4, 2):
        x = workload(1, H=4, S=700, decay="slow")
        x.q = np.ascontiguousarray(x.q[:, :, :Hk])
        x.k = np.ascontiguousarray(x.k[:, :, :Hk])
        do, dhT = make_cotangents(5, x)
        d = device_inputs(x)
        dO, dH = to_dev(do, torch.bfloat16), to_dev(dhT)
        run = lambda: gdn.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], dO, h0=d["h0"], dhT=dH)
        ref = run()
        torch.cuda.synchronize()
        g, out = capture(run)
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            for n, (a, b) in enumerate(zip(out, ref)):
                assert torch.equal(a, b), n
            run()                              # eager work between replays
            torch.cuda.synchronize()
