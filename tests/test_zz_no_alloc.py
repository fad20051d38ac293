"""gdn_forward_noalloc -- the forward for callers that cannot allocate (its
workspace is a device array inside the library) -- against gdn_forward with a
caller workspace, through the C ABI: the same kernels in the same order, so
the results must be bit-identical.  Two calls in a row, the second on a
smaller problem, both reusing the one scratch array; then a packed batch cut
into pieces."""
import numpy as np
import pytest
import torch

import chunked_gated_delta_gdn_amd as gdn
from chunked_gated_delta_gdn_amd import binding as b
from workloads import make_inputs, make_packed_inputs
from gpu_util import device_inputs, oracle_forward, check_forward, say

pytestmark = pytest.mark.gpu


def _both(x, n_segments=1, cu=None, m=0):
    d = device_inputs(x)
    q, k, v, g, beta, h0 = (d[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    p = gdn.problem_for(k, v, x.C, cu, n_segments, None, m)
    b.gdn_validate(p)
    N = len(cu) - 1 if cu is not None else k.shape[0]
    H, K, V = v.shape[2], k.shape[3], v.shape[3]
    need = b.gdn_forward_workspace_bytes(p)
    assert 0 < need <= b.GDN_FORWARD_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=v.device)
    o1 = torch.empty_like(v)
    h1 = torch.empty((N, H, K, V), dtype=torch.float32, device=v.device)
    o2 = torch.full_like(v, float("nan"))
    h2 = torch.full((N, H, K, V), float("nan"), dtype=torch.float32, device=v.device)
    st = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    b.gdn_forward(p, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(h0), ptr(o1), ptr(h1), ptr(ws), need, st)
    b.gdn_forward_noalloc(p, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(h0), ptr(o2), ptr(h2), st)
    torch.cuda.synchronize()
    return (o1, h1), (o2, h2), need


def test_noalloc_matches_gdn_forward_on_two_calls():
    # call 1: a 4k-token sequence in 4 segments, 8 heads (4 MiB of scratch)
    x1 = make_inputs(81, 1, 4096, 8, 128, 128, 64, "bf16", 0.02, "slow", name="noalloc-1")
    (o1, h1), (o2, h2), need1 = _both(x1, n_segments=4)
    say(f"  noalloc call 1: {need1} bytes of scratch")
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, h_ref = oracle_forward(x1)
    check_forward(x1, o2.float().cpu().numpy(), h2.cpu().numpy(), o_ref, h_ref, what="noalloc call 1")
    # call 2, smaller: 1000 tokens in 3 segments, 2 heads, the same scratch array
    x2 = make_inputs(82, 1, 1000, 2, 128, 128, 64, "bf16", 0.02, "slow", name="noalloc-2")
    (o1, h1), (o2, h2), need2 = _both(x2, n_segments=3)
    say(f"  noalloc call 2: {need2} bytes of scratch")
    assert need2 < need1
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, h_ref = oracle_forward(x2)
    check_forward(x2, o2.float().cpu().numpy(), h2.cpu().numpy(), o_ref, h_ref, what="noalloc call 2")


def test_noalloc_packed_pieces():
    x = make_packed_inputs(83, 4, 2500, 2, 128, 128, 64, "bf16", h0_std=0.02, decay="slow", median=400,
                           pad_to_chunk=False, name="noalloc-packed")
    cu = [int(c) for c in x.cu_seqlens]
    (o1, h1), (o2, h2), need = _both(x, cu=cu, m=3)
    say(f"  noalloc packed: {need} bytes of scratch")
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
