"""Negative controls on the GPU path: the parity check must reject a planted
mistake (the style of the negative controls on the Ulysses context-parallelism
page, section "Tests": tests that have to fail when the plumbing is wrong).

The segment pass runs through its public entry points -- the carrying scan
(gdn_scan GDN_SCAN_CARRY), the exclusive prefix scan (gdn_segment_compose) and
the emitting re-pass (gdn_scan GDN_SCAN_EMIT) -- and a mistake is planted on
the host between them: the transition M zeroed, replaced by the identity or
transposed, the incoming segment states permuted, or the prefix scan skipped.
The inputs have no decay (g = 0) and 256-token segments, so that M carries a
large share of every incoming state (under the workload decay M of a long
segment underflows to zero and no check could see it).  Unplanted, the same
pass is within tolerance."""
import numpy as np
import pytest
import torch

import chunked_gated_delta_gdn_amd as gdn
from workloads import make_inputs
from gpu_util import TOL, device_inputs, oracle_forward, say, check_forward, rel_err, slice_err

pytestmark = pytest.mark.gpu

R = 4


@pytest.fixture(scope="module")
def case():
    x = make_inputs(70, 1, 1024, 2, 128, 128, 64, "bf16", 0.02, "none", name="controls")
    o_ref, h_ref = oracle_forward(x)
    d = device_inputs(x)
    M, U = gdn.scan_carry(d["k"], d["v"], d["g"], d["beta"], chunk_size=64, n_segments=R)
    torch.cuda.synchronize()
    return x, d, M, U, o_ref, h_ref


def _finish(d, M, U, h_in=None):
    if h_in is None:
        h_in, _ = gdn.segment_compose(M, U, h0=d["h0"])
    o, hT = gdn.scan_emit(d["q"], d["k"], d["v"], d["g"], d["beta"], h_in=h_in, chunk_size=64,
                              n_segments=R)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), hT.cpu().numpy()


def test_unplanted_segment_pass_passes(case):
    x, d, M, U, o_ref, h_ref = case
    o, hT = _finish(d, M, U)
    check_forward(x, o, hT, o_ref, h_ref, what="unplanted")


def _plant(name, d, M, U):
    if name == "zero_M":
        return _finish(d, torch.zeros_like(M), U)
    if name == "identity_M":
        eye = torch.eye(M.shape[-1], device=M.device).expand_as(M).contiguous()
        return _finish(d, eye, U)
    if name == "transposed_M":
        return _finish(d, M.transpose(-1, -2).contiguous(), U)
    h_in, _ = gdn.segment_compose(M, U, h0=d["h0"])
    if name == "permuted_h_in":
        return _finish(d, M, U, h_in=h_in[[0, 2, 1, 3]].contiguous())
    if name == "compose_skipped":
        return _finish(d, M, U, h_in=d["h0"].expand_as(h_in).contiguous())
    raise ValueError(name)


@pytest.mark.parametrize("plant", ["zero_M", "identity_M", "transposed_M", "permuted_h_in", "compose_skipped"])
def test_planted_mistake_fails_the_check(case, plant):
    x, d, M, U, o_ref, h_ref = case
    o, hT = _plant(plant, d, M, U)
    eo, eh = rel_err(o, o_ref), rel_err(hT, h_ref)
    so = slice_err(o, o_ref, (0, 2))
    say(f"  planted {plant}: err(o)={eo:.3e} (worst head {so:.3e}) err(hT)={eh:.3e} tol={TOL['bf16']:g}")
    # the mistake must be caught, and by a wide margin: a check that passed it
    # would also pass a kernel with the same fault
    assert max(eo, eh, so) > 5 * TOL["bf16"]
    with pytest.raises(AssertionError):
        check_forward(x, o, hT, o_ref, h_ref, what=f"planted {plant}")
