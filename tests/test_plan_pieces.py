"""The packed-batch piece planner and the piece split rule (CPU only)."""
import pytest

from chunked_gated_delta_gdn_amd import binding as b
from chunked_gated_delta_gdn_amd import ops


def test_longest_sequence_of_the_packed_workload_is_cut():
    """8 sequences of 323, 4, 64, 24, 27, 34, 6, 34 chunks, 32 heads, 256 CUs:
    one chain per sequence would run 323 chunk steps; pieces finish sooner."""
    chunks = (323, 4, 64, 24, 27, 34, 6, 34)
    m = ops.plan_pieces(chunks, 32, 256)
    assert 0 < m < 323
    whole = ops._lpt_makespan([(c, 64) for c in chunks], 256)
    assert whole == 323


def test_balanced_batches_stay_whole():
    assert ops.plan_pieces((16,) * 64, 32, 256) == 0        # 4096 workgroups already fill the chip
    assert ops.plan_pieces((0,), 4, 256) == 0
    assert ops.plan_pieces((1, 1, 1), 2, 256) == 0


def test_long_single_sequence_is_cut():
    m = ops.plan_pieces((1024,), 32, 256)
    assert 0 < m < 1024


def test_too_many_pieces_are_never_planned():
    m = ops.plan_pieces((40,) * 200, 1, 256)
    if m:
        assert sum(len(ops._piece_chunks(40, m)) for _ in range(200)) <= b.GDN_MAX_SEQS


def test_lpt_makespan():
    assert ops._lpt_makespan([(10, 4)], 4) == 10
    assert ops._lpt_makespan([(10, 5)], 4) == 20
    assert ops._lpt_makespan([(10, 4), (3, 4)], 4) == 13
    assert ops._lpt_makespan([(0, 100)], 4) == 0


@pytest.mark.parametrize("nc", [1, 2, 7, 8, 9, 64, 65, 323, 1024])
@pytest.mark.parametrize("m", [1, 3, 8, 64, 100])
def test_split_rule_matches_the_library(nc, m):
    """ops._piece_chunks (the planner's model) cuts like the library: the same
    number of pieces, sizes summing to the sequence, no piece above m."""
    C = 16
    pcs = ops._piece_chunks(nc, m)
    if nc > 256 * m:
        return
    p = b.make_problem(1, nc * C, 1, 32, 32, C, b.GDN_F32, cu_seqlens=[0, nc * C], max_piece_chunks=m)
    assert b.gdn_num_pieces(p) == len(pcs)
    assert sum(pcs) == nc and max(pcs) <= max(m, 1) and min(pcs) >= 1
