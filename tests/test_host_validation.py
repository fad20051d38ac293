"""Host-side argument validation of the C ABI (CPU only: every case here is
rejected before anything touches a GPU)."""
import json
import os

import pytest

from chunked_gated_delta_gdn_amd import binding as b

FAKE = 0x7f0000000000        # a 16-byte aligned address that is never dereferenced
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def prob(**kw):
    args = dict(B=1, S=256, H=2, K=32, V=32, C=16, dtype=b.GDN_F32)
    args.update(kw)
    cu = args.pop("cu_seqlens", None)
    R = args.pop("n_segments", 1)
    ss = args.pop("seg_starts", None)
    return b.make_problem(cu_seqlens=cu, n_segments=R, seg_starts=ss, **args)


def status(p):
    return b.gdn_validate(p, raise_on_error=False)


def test_valid_problems():
    assert status(prob()) == b.GDN_OK
    assert status(prob(K=128, V=128, C=64, dtype=b.GDN_BF16, S=65536, H=32, n_segments=4)) == 0
    assert status(prob(S=0)) == b.GDN_OK
    assert status(prob(S=250, n_segments=4)) == b.GDN_OK
    assert status(prob(S=100, cu_seqlens=[0, 30, 30, 100])) == b.GDN_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(S=-1), dict(H=0), dict(K=0), dict(C=0)])
def test_bad_sizes(kw):
    assert status(prob(**kw)) == b.GDN_EINVAL


@pytest.mark.parametrize("kw", [dict(K=64, V=64, C=32), dict(C=32), dict(K=128, V=64, C=64),
                                dict(dtype=7)])
def test_unsupported_shapes(kw):
    assert status(prob(**kw)) == b.GDN_EUNSUPPORTED


@pytest.mark.parametrize("ss", [[0, 16, 8, 32], [0, 8, 32, 64], [16, 32, 48, 64],
                                [0, 64, 64, 128], [0, 64, 128, 256]])
def test_segments_must_be_contiguous_in_order_and_chunk_aligned(ss):
    """MaxText PR, section 'Limitation': a sequential recurrence needs contiguous,
    in-order slices; anything else is an error, never a silent wrong result."""
    assert status(prob(n_segments=4, seg_starts=ss)) == b.GDN_EORDER


def test_too_many_segments():
    assert status(prob(S=32, n_segments=3)) == b.GDN_EINVAL
    assert status(prob(S=4096, n_segments=b.GDN_MAX_SEGMENTS + 1)) == b.GDN_EUNSUPPORTED


def test_packed_mode_rules():
    assert status(prob(S=100, cu_seqlens=[0, 60, 50, 100])) == b.GDN_EORDER
    assert status(prob(S=100, cu_seqlens=[5, 60, 100])) == b.GDN_EORDER
    assert status(prob(S=100, cu_seqlens=[0, 60, 90])) == b.GDN_EINVAL
    assert status(prob(S=100, B=2, cu_seqlens=[0, 100])) == b.GDN_EINVAL
    assert status(prob(S=100, cu_seqlens=[0, 100], n_segments=2)) == b.GDN_EUNSUPPORTED
    many = list(range(0, b.GDN_MAX_SEQS + 2))
    assert status(prob(S=many[-1], cu_seqlens=many)) == b.GDN_EUNSUPPORTED


def test_wy_workspace_must_hold_the_problem():
    """A WY workspace smaller than gdn_wy_workspace_bytes is GDN_EWORKSPACE for
    gdn_chunk_prepare and for every scan mode, before anything is launched
    (the pointers here are never dereferenced); wy = NULL ignores wy_bytes."""
    import ctypes
    lib = b.library()
    for p in (prob(S=250, B=3), prob(K=128, V=128, C=64, dtype=b.GDN_BF16, S=1000, H=4, n_segments=3),
              prob(S=100, cu_seqlens=[0, 17, 17, 100], dtype=b.GDN_BF16, max_piece_chunks=2)):
        need = b.gdn_wy_workspace_bytes(p)
        assert need > 0
        assert lib.gdn_chunk_prepare(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
            b.GDN_EWORKSPACE
        assert lib.gdn_chunk_prepare(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == b.GDN_EWORKSPACE
        modes = [b.GDN_SCAN_EMIT, b.GDN_SCAN_CARRY]
        modes += [b.GDN_SCAN_HEAD_EMIT_CARRY] if p.n_seqs or p.n_segments > 1 else []
        modes += [b.GDN_SCAN_TAIL_EMIT] if p.n_seqs else []
        for mode in modes:
            full = dict(M=FAKE, U=FAKE, h_out=FAKE + (1 << 30))
            assert _scan_status(p, mode, wy=FAKE, wy_bytes=need - 16, **full) == b.GDN_EWORKSPACE, mode
            assert _scan_status(p, mode, wy=FAKE, wy_bytes=0, **full) == b.GDN_EWORKSPACE, mode
            # no workspace: wy_bytes is not looked at (the call then fails later,
            # at the launch, because this machine has no GPU -- but not on size)
            assert _scan_status(p, mode, wy=None, wy_bytes=0, **full) != b.GDN_EWORKSPACE, mode
    assert "GDN_EWORKSPACE" in lib.gdn_status_string(b.GDN_EWORKSPACE).decode()


def test_chunk_rows_must_span_less_than_2gib():
    """The kernels reach the C rows of a chunk through 32-bit byte offsets from
    the chunk's first row: problems whose C rows of q, k or of v, o span 2 GiB
    or more are GDN_EUNSUPPORTED instead of silently reading zeros."""
    big = dict(K=128, V=128, C=64, dtype=b.GDN_BF16, S=64)
    assert status(prob(H=131071, **big)) == b.GDN_OK              # 64 * 131071 * 256 B < 2 GiB
    assert status(prob(H=131072, **big)) == b.GDN_EUNSUPPORTED    # = 2 GiB
    assert status(prob(H=131072, H_qk=1, **big)) == b.GDN_EUNSUPPORTED   # v, o rows alone
    assert status(prob(H=65536, **dict(big, dtype=b.GDN_F32))) == b.GDN_EUNSUPPORTED
    assert status(prob(H=65535, **dict(big, dtype=b.GDN_F32))) == b.GDN_OK
    # and the scan refuses it before any launch
    assert _scan_status(prob(H=131072, **big)) == b.GDN_EUNSUPPORTED


def test_workspace_sizes():
    p = prob(S=250, B=3)                      # 16 chunks per sequence, ragged tail
    assert b.gdn_wy_workspace_bytes(p) == 3 * 16 * 2 * 16 * (32 + 32) * 4
    p = prob(S=100, cu_seqlens=[0, 17, 17, 100], dtype=b.GDN_BF16)   # 2 + 0 + 6 chunks
    assert b.gdn_wy_workspace_bytes(p) == 8 * 2 * 16 * 64 * 2
    assert b.gdn_wy_workspace_bytes(prob(C=5)) == 0


def test_segment_payload_is_sequence_length_independent():
    """The (M_r, U_r) payload is cp*B*H*K*(K+V) fp32 elements whatever S is
    (MaxText PR, sections 'Tests' and 'Measured results')."""
    with open(os.path.join(GOLDEN, "segment_payload.json")) as f:
        d = json.load(f)
    elems = 1
    for x in d["hlo_shape"]:
        elems *= x
    assert elems == d["cp"] * d["BH"] * d["K"] * (d["K"] + d["V"])
    sizes = set()
    for S in d["seq_lens"]:
        p = prob(B=1, H=d["BH"], S=S, K=d["K"], V=d["V"], C=64, n_segments=d["cp"])
        sizes.add(b.gdn_segment_workspace_bytes(p))
    assert sizes == {elems * 4}


def _scan_status(p, mode=b.GDN_SCAN_EMIT, **ptrs):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, wy=None, h_in=None, o=FAKE,
                h_out=None, M=None, U=None)
    args.update(ptrs)
    wy_bytes = args.pop("wy_bytes", b.gdn_wy_workspace_bytes(p))
    lib = b.library()
    import ctypes
    return lib.gdn_scan(ctypes.byref(p), mode, args["q"], args["k"], args["v"], args["g"],
                        args["beta"], args["wy"], wy_bytes, args["h_in"], args["o"], args["h_out"],
                        args["M"], args["U"], None)


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "o"])
def test_scan_rejects_null_inputs(name):
    assert _scan_status(prob(), **{name: None}) == b.GDN_EINVAL


@pytest.mark.parametrize("name", ["q", "k", "g", "o", "h_in", "wy"])
def test_scan_rejects_misaligned_pointers(name):
    assert _scan_status(prob(), **{name: FAKE + 4}) == b.GDN_EINVAL


def test_scan_rejects_bad_mode_and_missing_carry_outputs():
    assert _scan_status(prob(), mode=5) == b.GDN_EINVAL
    assert _scan_status(prob(), mode=b.GDN_SCAN_CARRY) == b.GDN_EINVAL
    assert _scan_status(prob(), mode=b.GDN_SCAN_CARRY, M=FAKE) == b.GDN_EINVAL


def test_head_emit_carry_mode_rules():
    """GDN_SCAN_HEAD_EMIT_CARRY needs batch mode, at least two segments, the
    carried pairs and the emitting pass's q and o."""
    H = b.GDN_SCAN_HEAD_EMIT_CARRY
    full = dict(M=FAKE, U=FAKE)
    assert _scan_status(prob(n_segments=1), mode=H, **full) == b.GDN_EINVAL
    # packed: the carried middle pieces need M and U
    assert _scan_status(prob(S=100, cu_seqlens=[0, 30, 100], max_piece_chunks=1), mode=H) == b.GDN_EINVAL
    assert _scan_status(prob(n_segments=3), mode=H) == b.GDN_EINVAL
    assert _scan_status(prob(n_segments=3), mode=H, M=FAKE) == b.GDN_EINVAL
    assert _scan_status(prob(n_segments=3), mode=H, q=None, **full) == b.GDN_EINVAL
    assert _scan_status(prob(n_segments=3), mode=H, o=None, **full) == b.GDN_EINVAL
    assert _scan_status(prob(n_segments=3), mode=H, h_out=FAKE + 4, **full) == b.GDN_EINVAL


def test_packed_piece_rules():
    """Pieces: packed problems only, a non-negative cap, at most GDN_MAX_SEQS of
    them; the tail mode is packed-only and its states are per piece."""
    assert status(prob(S=100, cu_seqlens=[0, 30, 100], max_piece_chunks=-1)) == b.GDN_EINVAL
    assert status(prob(max_piece_chunks=2)) == b.GDN_EINVAL
    assert status(prob(S=16 * 300, cu_seqlens=[0, 16 * 300], max_piece_chunks=1)) == b.GDN_EUNSUPPORTED
    assert status(prob(S=16 * 300, cu_seqlens=[0, 16 * 300], max_piece_chunks=2)) == b.GDN_OK
    assert status(prob(S=100, cu_seqlens=[0, 30, 100], max_piece_chunks=1, n_segments=2)) == b.GDN_EUNSUPPORTED
    T = b.GDN_SCAN_TAIL_EMIT
    assert _scan_status(prob(n_segments=2), mode=T, h_in=FAKE) == b.GDN_EINVAL
    # per-piece h_in spans P > N states: h_out may not alias it
    pk = prob(S=100, cu_seqlens=[0, 30, 100], max_piece_chunks=2)
    assert _scan_status(pk, mode=T, h_in=FAKE, h_out=FAKE) == b.GDN_EINVAL
    assert _scan_status(pk, mode=b.GDN_SCAN_EMIT, h_in=FAKE, h_out=FAKE) == b.GDN_EINVAL


@pytest.mark.parametrize("cu,m,expect", [([0, 30, 30, 100], 0, 3), ([0, 30, 30, 100], 2, 5),
                                          ([0, 30, 30, 100], 5, 3), ([0, 30, 30, 100], 4, 4),
                                          ([0, 256], 3, 6), ([0, 0], 1, 1)])
def test_num_pieces(cu, m, expect):
    """Chunks per sequence at C = 16: [0,30,30,100] -> 2, 0, 5; a sequence of
    c > m chunks makes ceil(c / m) pieces, every other sequence one."""
    p = prob(S=cu[-1], cu_seqlens=cu, max_piece_chunks=m)
    assert b.gdn_num_pieces(p) == expect
    assert b.gdn_segment_workspace_bytes(p) == expect * 2 * 32 * 64 * 4


def test_num_pieces_batch_and_invalid():
    assert b.gdn_num_pieces(prob(B=3, n_segments=4)) == 12
    assert b.gdn_num_pieces(prob(B=0)) == -1


def test_piece_compose_validation():
    import ctypes
    lib = b.library()
    pk = prob(S=100, cu_seqlens=[0, 30, 100], max_piece_chunks=2)
    ref = ctypes.byref
    assert lib.gdn_piece_compose(ref(prob(n_segments=2)), 0, FAKE, FAKE, None, FAKE, None, None) == b.GDN_EINVAL
    assert lib.gdn_piece_compose(ref(pk), 2, FAKE, FAKE, None, FAKE, None, None) == b.GDN_EINVAL
    assert lib.gdn_piece_compose(ref(pk), 0, None, FAKE, None, FAKE, None, None) == b.GDN_EINVAL
    assert lib.gdn_piece_compose(ref(pk), 0, FAKE, FAKE, None, None, None, None) == b.GDN_EINVAL
    # h_in aliasing M, h_final aliasing h_in
    assert lib.gdn_piece_compose(ref(pk), 0, FAKE, FAKE + (1 << 30), None, FAKE, None, None) == b.GDN_EINVAL
    assert lib.gdn_piece_compose(ref(pk), 0, FAKE, FAKE + (1 << 30), None, FAKE + (1 << 31), FAKE + (1 << 31),
                                 None) == b.GDN_EINVAL
    # first = 1 with every sequence one piece long reads nothing and writes no h_in
    one = prob(S=100, cu_seqlens=[0, 30, 100])
    assert lib.gdn_piece_compose(ref(pk), 1, None, None, None, None, None, None) == b.GDN_EINVAL
    assert lib.gdn_piece_compose(ref(one), 1, None, None, None, None, None, None) == b.GDN_OK


def test_scan_rejects_state_alias_with_segments():
    p = prob(n_segments=4)
    assert _scan_status(p, h_in=FAKE, h_out=FAKE) == b.GDN_EINVAL


def test_error_messages_name_the_problem():
    st = _scan_status(prob(n_segments=4, seg_starts=[0, 32, 16, 64]))
    assert st == b.GDN_EORDER
    assert b"contiguous and in order" in b.library().gdn_last_error()


def test_compose_and_decode_validation():
    lib = b.library()
    assert lib.gdn_segment_compose(0, 1, 1, 32, 32, FAKE, FAKE, None, FAKE, None, None) == b.GDN_EINVAL
    assert lib.gdn_segment_compose(2, 1, 1, 64, 64, FAKE, FAKE, None, FAKE, None, None) == b.GDN_EUNSUPPORTED
    assert lib.gdn_segment_compose(2, 1, 1, 32, 32, FAKE, FAKE, None, None, None, None) == b.GDN_EINVAL
    # h_in aliasing M is refused
    assert lib.gdn_segment_compose(2, 1, 1, 32, 32, FAKE, FAKE + (1 << 20), None, FAKE, None,
                                   None) == b.GDN_EINVAL
    assert lib.gdn_decode_step(4, 2, 2, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_EUNSUPPORTED
    assert lib.gdn_decode_step(4, 2, 2, 32, 32, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_EUNSUPPORTED
    assert lib.gdn_decode_step(4, 2, 2, 32, 32, 0, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_EINVAL
    assert lib.gdn_decode_step(4, 0, 1, 32, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_EINVAL
    assert lib.gdn_decode_step(0, 2, 2, 32, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_OK
    # grouped heads: H_qk must divide H
    for hq in (0, 4, 12, -1):
        assert lib.gdn_decode_step(4, 6, hq, 32, 32, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_EINVAL


@pytest.mark.parametrize("hq,ok", [(0, True), (1, True), (2, True), (4, True), (3, False), (8, False), (-1, False)])
def test_grouped_heads_rules(hq, ok):
    """q, k may have H_qk heads for H = 4 value heads when H_qk divides H
    (0 means H_qk = H)."""
    st = status(prob(H=4, H_qk=hq))
    assert st == (b.GDN_OK if ok else b.GDN_EINVAL)


def test_conv_and_norm_validation():
    import ctypes
    lib = b.library()
    conv = lambda *a: lib.gdn_causal_conv1d(*a)
    assert conv(2, 16, 8, 0, b.GDN_F32, 1, None, 0, FAKE, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EINVAL
    assert conv(2, 16, 8, 9, b.GDN_F32, 1, None, 0, FAKE, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EINVAL
    assert conv(2, 16, 8, 4, 7, 1, None, 0, FAKE, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EUNSUPPORTED
    assert conv(2, 16, 8, 4, b.GDN_F32, 2, None, 0, FAKE, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EINVAL
    assert conv(2, 16, 8, 4, b.GDN_F32, 1, None, 0, FAKE, FAKE, None, None, FAKE, None) == b.GDN_EINVAL   # y == x
    assert conv(2, 16, 8, 4, b.GDN_F32, 1, None, 0, None, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EINVAL
    cu = (ctypes.c_int32 * 3)(0, 20, 10)
    assert conv(1, 10, 8, 4, b.GDN_F32, 1, cu, 2, FAKE, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EORDER
    cu = (ctypes.c_int32 * 3)(0, 5, 12)
    assert conv(2, 12, 8, 4, b.GDN_F32, 1, cu, 2, FAKE, FAKE, None, None, FAKE + (1 << 20), None) == b.GDN_EINVAL
    # in-place state with a sequence crossing token 64
    assert conv(1, 100, 8, 4, b.GDN_F32, 1, None, 0, FAKE, FAKE, FAKE + (2 << 20), FAKE + (2 << 20),
                FAKE + (1 << 20), None) == b.GDN_EINVAL
    norm = lib.gdn_gated_rmsnorm
    assert norm(4, 0, b.GDN_F32, 1e-6, FAKE, None, FAKE, FAKE, None) == b.GDN_EINVAL
    assert norm(4, 257, b.GDN_F32, 1e-6, FAKE, None, FAKE, FAKE, None) == b.GDN_EINVAL
    assert norm(4, 128, b.GDN_F32, -1.0, FAKE, None, FAKE, FAKE, None) == b.GDN_EINVAL
    assert norm(4, 128, 5, 1e-6, FAKE, None, FAKE, FAKE, None) == b.GDN_EUNSUPPORTED
    assert norm(4, 128, b.GDN_F32, 1e-6, FAKE, None, None, FAKE, None) == b.GDN_EINVAL
    assert norm(4, 128, b.GDN_F32, 1e-6, FAKE, None, FAKE, FAKE + 16, None) == b.GDN_EINVAL   # partial overlap
    assert norm(0, 128, b.GDN_F32, 1e-6, None, None, None, None, None) == b.GDN_OK


def test_backward_validation():
    """gdn_backward: every buffer distinct, the workspace sized by
    gdn_backward_workspace_bytes (growing by the carries and boundary states
    of chains that split sequences)."""
    import ctypes
    lib = b.library()
    ref = ctypes.byref
    p = prob()                                    # B1 S256 H2 K32 V32 C16 fp32
    ws = b.gdn_backward_workspace_bytes(p)
    assert ws == 16 * 2 * 4 * (3 * 16 * 16 + 16 * 32 + 3 * 16 * 32 + 2 * 32 * 32)
    # segments and pieces: per chain and head M, Mt [K,K] and U, E, h_in, dh_in [K,V]
    per_chain = 2 * 4 * (2 * 32 * 32 + 4 * 32 * 32)
    assert b.gdn_backward_workspace_bytes(prob(n_segments=2)) == ws + 2 * per_chain
    assert b.gdn_backward_workspace_bytes(prob(B=3, n_segments=4)) == 3 * ws + 12 * per_chain
    assert b.gdn_backward_workspace_bytes(prob(n_segments=2, seg_starts=[0, 100])) == 0   # invalid as given
    # packed: 3 chunks + 8 chunks at m = 2 -> 2 + 4 pieces
    pk = prob(S=176, cu_seqlens=[0, 48, 176], max_piece_chunks=2)
    pk0 = prob(S=176, cu_seqlens=[0, 48, 176])
    assert b.gdn_backward_workspace_bytes(pk) == b.gdn_backward_workspace_bytes(pk0) + 6 * per_chain
    # grouped key heads add fp32 dq, dk rows of every value head
    wg = b.gdn_backward_workspace_bytes(prob(H=4, H_qk=2))
    assert wg == 2 * ws + 2 * 256 * 4 * 32 * 4
    step = 1 << 24                                # distinct fake buffers, 16 MiB apart
    buf = [FAKE + i * step for i in range(16)]

    def call(pp, **over):
        names = ["q", "k", "v", "g", "beta", "h0", "dout", "dhT", "dq", "dk", "dv", "dg", "dbeta", "dh0",
                 "ws"]
        a = dict(zip(names, buf))
        a.update(over)
        return lib.gdn_backward(ref(pp), *[a[n] for n in names], over.get("ws_bytes", ws), None)

    assert call(prob(H=4, H_qk=2), ws_bytes=wg - 1) == b.GDN_EWORKSPACE
    assert call(prob(S=100, cu_seqlens=[0, 30, 100], max_piece_chunks=-1)) == b.GDN_EINVAL
    assert call(p, ws_bytes=ws - 1) == b.GDN_EWORKSPACE
    assert call(prob(n_segments=2), ws_bytes=ws + 2 * per_chain - 1) == b.GDN_EWORKSPACE
    assert call(p, q=None) == b.GDN_EINVAL
    assert call(p, dout=None) == b.GDN_EINVAL
    assert call(p, dg=buf[1] + 4) == b.GDN_EINVAL          # misaligned
    assert call(p, dq=buf[0]) == b.GDN_EINVAL              # dq overlaps q
    assert call(p, dk=buf[14]) == b.GDN_EINVAL             # dk overlaps the workspace
    assert call(p, dv=buf[8]) == b.GDN_EINVAL              # dv overlaps dq
    assert call(prob(K=64, V=64, C=16)) == b.GDN_EUNSUPPORTED


def test_forward_workspace_and_checks():
    """gdn_forward: workspace sized by gdn_forward_workspace_bytes (none for one
    chain per sequence), GDN_EWORKSPACE when short, no overlap of the workspace
    with o, h0 or h_out, and the usual pointer checks -- all before a launch."""
    import ctypes
    lib = b.library()
    sv = 2 * 32 * 32 * 4                       # H K V fp32
    assert b.gdn_forward_workspace_bytes(prob()) == 0
    # batch R = 4, B = 3: h1 [3] | M [2,3] | U [2,3] | h_all [3,3] state rows (K = V)
    assert b.gdn_forward_workspace_bytes(prob(B=3, n_segments=4)) == (3 + 6 + 6 + 9) * sv
    assert b.gdn_forward_workspace_bytes(prob(B=3, n_segments=2)) == (3 + 0 + 0 + 3) * sv
    # packed: 3 chunks + 8 chunks at m = 2 -> 2 + 4 pieces; hs [2] | M, U, h_in [6]
    pk = prob(S=176, cu_seqlens=[0, 48, 176], max_piece_chunks=2)
    assert b.gdn_num_pieces(pk) == 6
    assert b.gdn_forward_workspace_bytes(pk) == (2 + 3 * 6) * sv
    assert b.gdn_forward_workspace_bytes(prob(S=176, cu_seqlens=[0, 48, 176])) == 0
    step = 1 << 24
    buf = [FAKE + i * step for i in range(12)]

    def call(pp, ws_bytes=None, **over):
        names = ["q", "k", "v", "g", "beta", "h0", "o", "h_out", "ws"]
        a = dict(zip(names, buf))
        a.update(over)
        n = b.gdn_forward_workspace_bytes(pp) if ws_bytes is None else ws_bytes
        return lib.gdn_forward(ctypes.byref(pp), *[a[x] for x in names], n, None)

    p4 = prob(n_segments=4)
    need = b.gdn_forward_workspace_bytes(p4)
    assert call(p4, ws_bytes=need - 1) == b.GDN_EWORKSPACE
    assert call(pk, ws_bytes=0) == b.GDN_EWORKSPACE
    assert call(p4, ws=None) == b.GDN_EINVAL
    assert call(p4, ws=buf[6]) == b.GDN_EINVAL           # overlaps o
    assert call(p4, ws=buf[5] + 4096) == b.GDN_EINVAL     # overlaps h0 (8 KiB)
    assert call(p4, ws=buf[7] - 4096) == b.GDN_EINVAL     # overlaps h_out
    assert call(p4, q=None) == b.GDN_EINVAL
    assert call(p4, o=buf[6] + 8) == b.GDN_EINVAL         # misaligned
    assert call(prob(K=64, V=64, C=32, n_segments=4)) == b.GDN_EUNSUPPORTED
    assert call(prob(n_segments=4, seg_starts=[0, 32, 16, 64])) == b.GDN_EORDER


def test_forward_noalloc_rejects_problems_beyond_its_scratch():
    """gdn_forward_noalloc holds a fixed scratch array: a problem whose
    workspace exceeds it is GDN_EWORKSPACE before anything is launched (the
    pointers here are never dereferenced)."""
    import ctypes
    lib = b.library()
    big = prob(K=128, V=128, C=64, dtype=b.GDN_BF16, S=64 * 64, H=64, n_segments=64)
    assert b.gdn_forward_workspace_bytes(big) > b.GDN_FORWARD_SCRATCH_BYTES
    assert lib.gdn_forward_noalloc(ctypes.byref(big), *([FAKE + (i << 28) for i in range(8)]), None) == \
        b.GDN_EWORKSPACE
    assert "64" in lib.gdn_last_error().decode() or "scratch" in lib.gdn_last_error().decode()
    # the 64k-token, 32-head forward in 4 segments fits (16 MiB)
    head = prob(K=128, V=128, C=64, dtype=b.GDN_BF16, S=65536, H=32, n_segments=4)
    assert b.gdn_forward_workspace_bytes(head) == 16 << 20
    assert lib.gdn_forward_noalloc(ctypes.byref(big), *([FAKE] * 5), None, FAKE, None, None) == b.GDN_EWORKSPACE
    assert lib.gdn_forward_noalloc(ctypes.byref(head), None, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None) == \
        b.GDN_EINVAL
