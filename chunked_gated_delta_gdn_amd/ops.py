"""Tensor-level calls of the library (PyTorch supplies device memory and streams).

Each function checks shapes and dtypes, allocates the outputs with torch and
forwards device addresses to the C entry point of the same name.  ``forward``
chains the entry points exactly as the three-phase pass of the MaxText PR "Add
context parallelism to the Gated Delta Net" (section "Implementation")
describes: one segment runs a single emitting scan; several segments run the
carrying scan (phase 1), the exclusive segment scan (phase 2) and the emitting
scan from the true incoming states (phase 3).
"""
import torch

from . import binding as _b

__all__ = ["problem_for", "chunk_prepare", "scan_emit", "scan_carry", "segment_compose",
           "segment_bounds", "forward_segmented",
           "decode_step", "forward"]


def _dtype_code(t):
    if t.dtype == torch.float32:
        return _b.GDN_F32
    if t.dtype == torch.bfloat16:
        return _b.GDN_BF16
    raise ValueError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _addr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def problem_for(k, v, chunk_size, cu_seqlens=None, n_segments=1, seg_starts=None):
    """The ``gdn_problem`` of batch tensors k [B,S,H,K], v [B,S,H,V]."""
    B, S, H, K = k.shape
    V = v.shape[-1]
    return _b.make_problem(B, S, H, K, V, chunk_size, _dtype_code(k), cu_seqlens=cu_seqlens,
                           n_segments=n_segments, seg_starts=seg_starts)


def _n_seqs(k, cu_seqlens):
    return k.shape[0] if cu_seqlens is None else len(cu_seqlens) - 1


def _check_inputs(q, k, v, g, beta):
    dev = k.device
    B, S, H, K = k.shape
    V = v.shape[-1]
    if q is not None:
        _need(q, "q", (B, S, H, K), k.dtype, dev)
    _need(k, "k", (B, S, H, K), k.dtype, dev)
    _need(v, "v", (B, S, H, V), k.dtype, dev)
    _need(g, "g", (B, S, H), torch.float32, dev)
    _need(beta, "beta", (B, S, H), torch.float32, dev)
    return B, S, H, K, V


def chunk_prepare(k, v, g, beta, chunk_size=64, cu_seqlens=None):
    """WY factors of every chunk (``gdn_chunk_prepare``): returns the workspace
    tensor (w blocks [n_chunks,H,C,K] then u blocks [n_chunks,H,C,V], in the
    input dtype) flattened to one dimension."""
    _check_inputs(None, k, v, g, beta)
    p = problem_for(k, v, chunk_size, cu_seqlens)
    _b.gdn_validate(p)
    nbytes = _b.gdn_wy_workspace_bytes(p)
    wy = torch.empty(nbytes // k.element_size(), dtype=k.dtype, device=k.device)
    _b.gdn_chunk_prepare(p, _addr(k), _addr(v), _addr(g), _addr(beta), _addr(wy),
                         _stream(k.device))
    return wy


def split_wy(wy, k, v, chunk_size, cu_seqlens=None):
    """Views (w [n_chunks,H,C,K], u [n_chunks,H,C,V]) of a WY workspace."""
    H, K, V = k.shape[2], k.shape[3], v.shape[3]
    n_chunks = wy.numel() // (H * chunk_size * (K + V))
    w = wy[: n_chunks * H * chunk_size * K].view(n_chunks, H, chunk_size, K)
    u = wy[n_chunks * H * chunk_size * K:].view(n_chunks, H, chunk_size, V)
    return w, u


def scan_emit(q, k, v, g, beta, h_in=None, wy=None, chunk_size=64, cu_seqlens=None,
              n_segments=1, seg_starts=None, output_final_state=True, out=None):
    """Emitting scan (``gdn_scan`` with GDN_SCAN_EMIT): returns (o, h_out).

    h_in is [N,H,K,V] for one segment, or [R,N,H,K,V] (the state entering each
    segment) for R segments; None means zero state everywhere."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    N = _n_seqs(k, cu_seqlens)
    p = problem_for(k, v, chunk_size, cu_seqlens, n_segments, seg_starts)
    _b.gdn_validate(p)
    if h_in is not None:
        shape = (N, H, K, V) if n_segments == 1 else (n_segments, N, H, K, V)
        _need(h_in, "h_in", shape, torch.float32, dev)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    o = out if out is not None else torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, S, H, V), k.dtype, dev)
    h_out = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    _b.gdn_scan(p, _b.GDN_SCAN_EMIT, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), _addr(h_in), _addr(o), _addr(h_out), None, None, _stream(dev))
    return o, h_out


def scan_head_carry(q, k, v, g, beta, h_in=None, wy=None, chunk_size=64, n_segments=2, seg_starts=None,
                    out=None):
    """Segment 0 emitted, segments 1 .. R-1 carried (``gdn_scan`` with
    GDN_SCAN_HEAD_EMIT_CARRY): returns (o, h1, M [R-1,B,H,K,K], U [R-1,B,H,K,V]).
    o holds segment 0's outputs (other tokens untouched when ``out`` is given),
    h1 [B,H,K,V] is segment 0's final state, the state entering segment 1."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    p = problem_for(k, v, chunk_size, None, n_segments, seg_starts)
    _b.gdn_validate(p)
    if h_in is not None:
        _need(h_in, "h_in", (B, H, K, V), torch.float32, dev)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    o = out if out is not None else torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, S, H, V), k.dtype, dev)
    h1 = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    M = torch.empty((n_segments - 1, B, H, K, K), dtype=torch.float32, device=dev)
    U = torch.empty((n_segments - 1, B, H, K, V), dtype=torch.float32, device=dev)
    _b.gdn_scan(p, _b.GDN_SCAN_HEAD_EMIT_CARRY, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), _addr(h_in), _addr(o), _addr(h1), _addr(M), _addr(U), _stream(dev))
    return o, h1, M, U


def scan_carry(k, v, g, beta, wy=None, chunk_size=64, n_segments=1, seg_starts=None):
    """Carrying zero-state scan (``gdn_scan`` with GDN_SCAN_CARRY): returns
    (M [R,B,H,K,K], U [R,B,H,K,V]) with h_end = M h_start + U per segment."""
    B, S, H, K, V = _check_inputs(None, k, v, g, beta)
    dev = k.device
    p = problem_for(k, v, chunk_size, None, n_segments, seg_starts)
    _b.gdn_validate(p)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    M = torch.empty((n_segments, B, H, K, K), dtype=torch.float32, device=dev)
    U = torch.empty((n_segments, B, H, K, V), dtype=torch.float32, device=dev)
    _b.gdn_scan(p, _b.GDN_SCAN_CARRY, None, _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), None, None, None, _addr(M), _addr(U), _stream(dev))
    return M, U


def segment_compose(M, U, h0=None, want_final=False):
    """Exclusive scan over segment pairs (``gdn_segment_compose``): returns
    (h_in [R,N,H,K,V], h_final [N,H,K,V] or None)."""
    R, N, H, K, _ = M.shape
    V = U.shape[-1]
    dev = M.device
    _need(M, "M", (R, N, H, K, K), torch.float32, dev)
    _need(U, "U", (R, N, H, K, V), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (N, H, K, V), torch.float32, dev)
    h_in = torch.empty((R, N, H, K, V), dtype=torch.float32, device=dev)
    h_final = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if want_final else None
    _b.gdn_segment_compose(R, N, H, K, V, _addr(M), _addr(U), _addr(h0), _addr(h_in),
                           _addr(h_final), _stream(dev))
    return h_in, h_final


def decode_step(q, k, v, g, beta, state, out=None):
    """One recurrent step (``gdn_decode_step``), updating ``state`` in place.

    q, k [B,H,K]; v [B,H,V]; g, beta [B,H] fp32; state [B,H,K,V] fp32.
    Returns o [B,H,V]."""
    B, H, K = k.shape
    V = v.shape[-1]
    dev = k.device
    _need(q, "q", (B, H, K), k.dtype, dev)
    _need(v, "v", (B, H, V), k.dtype, dev)
    _need(g, "g", (B, H), torch.float32, dev)
    _need(beta, "beta", (B, H), torch.float32, dev)
    _need(state, "state", (B, H, K, V), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, H, V), k.dtype, dev)
    _b.gdn_decode_step(B, H, K, V, _dtype_code(k), _addr(q), _addr(k), _addr(v), _addr(g),
                       _addr(beta), _addr(state), _addr(o), _stream(dev))
    return o


def segment_bounds(S, chunk_size, n_segments, seg_starts=None):
    """Token offsets of the segments and the end: the library's split when
    seg_starts is None (chunk r*n_chunks//R starts segment r)."""
    if seg_starts is not None:
        return [int(x) for x in seg_starts] + [S]
    nc = -(-S // chunk_size)
    return [(r * nc // n_segments) * chunk_size for r in range(n_segments)] + [S]


def _untimed(_name, fn):
    return fn()


def forward_segmented(q, k, v, g, beta, h0=None, chunk_size=64, n_segments=2, seg_starts=None,
                      output_final_state=True, timer=_untimed):
    """The three-phase segment pass on one sequence (B == 1), without its two
    redundant pieces: segment 0 starts from the true initial state, so it needs
    no carried M and is emitted directly (its final state is the state entering
    segment 1); the last segment is emitted from its incoming state, so it needs
    no carrying pass.  One launch emits segment 0 beside the carrying pass of
    segments 1 .. R-2 (GDN_SCAN_HEAD_EMIT_CARRY); then the segment scan seeded
    with segment 0's final state; then the emitting pass of segments 1 .. R-1.

    ``timer(name, fn)`` wraps each launch (for per-kernel timing)."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    if B != 1:
        raise ValueError("forward_segmented takes one sequence (B == 1)")
    R = n_segments
    _b.gdn_validate(problem_for(k, v, chunk_size, None, R, seg_starts))
    dev = k.device
    if h0 is not None:
        _need(h0, "h0", (B, H, K, V), torch.float32, dev)
    bnd = segment_bounds(S, chunk_size, R, seg_starts)
    s1, sl = bnd[1], bnd[R - 1]
    o = torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    if R > 2:
        head = slice(0, sl)
        _, h1, M, U = timer("scan_head_carry", lambda: scan_head_carry(
            q[:, head], k[:, head], v[:, head], g[:, head], beta[:, head], h_in=h0,
            chunk_size=chunk_size, n_segments=R - 1, seg_starts=bnd[:R - 1], out=o[:, head]))
        # states entering segments 1 .. R-1: the scan's outputs, then its final state
        h_all = torch.empty((R - 1, B, H, K, V), dtype=torch.float32, device=dev)
        timer("segment_compose", lambda: _b.gdn_segment_compose(
            R - 2, B, H, K, V, _addr(M), _addr(U), _addr(h1), _addr(h_all), _addr(h_all[R - 2]),
            _stream(dev)))
    else:
        first = slice(0, s1)
        _, h_all = timer("scan_emit_first", lambda: scan_emit(
            q[:, first], k[:, first], v[:, first], g[:, first], beta[:, first], h_in=h0,
            chunk_size=chunk_size, out=o[:, first]))
    rest = slice(s1, S)
    _, hT = timer("scan_emit", lambda: scan_emit(
        q[:, rest], k[:, rest], v[:, rest], g[:, rest], beta[:, rest], h_in=h_all,
        chunk_size=chunk_size, n_segments=R - 1, seg_starts=[b - s1 for b in bnd[1:R]],
        output_final_state=output_final_state, out=o[:, rest]))
    return o, hT


def forward(q, k, v, g, beta, h0=None, chunk_size=64, cu_seqlens=None, n_segments=1,
            seg_starts=None, reuse_wy=False, output_final_state=True, schedule="auto"):
    """Chunked gated delta rule forward: returns (o, final state or None).

    n_segments > 1 runs the three-phase segment pass; reuse_wy prepares the WY
    factors once (``gdn_chunk_prepare``) and hands them to both scans instead of
    recomputing them inside each scan.  schedule="auto" uses forward_segmented
    for one sequence with recomputed WY factors, "plain" always runs the full
    carrying pass over every segment."""
    if schedule not in ("auto", "plain"):
        raise ValueError(f"unknown schedule {schedule!r}")
    if (schedule == "auto" and n_segments > 1 and cu_seqlens is None and not reuse_wy
            and k.shape[0] == 1):
        return forward_segmented(q, k, v, g, beta, h0=h0, chunk_size=chunk_size,
                                 n_segments=n_segments, seg_starts=seg_starts,
                                 output_final_state=output_final_state)
    wy = chunk_prepare(k, v, g, beta, chunk_size, cu_seqlens) if reuse_wy else None
    if n_segments == 1:
        return scan_emit(q, k, v, g, beta, h_in=h0, wy=wy, chunk_size=chunk_size,
                         cu_seqlens=cu_seqlens, output_final_state=output_final_state)
    if cu_seqlens is not None:
        raise ValueError("segments are not supported together with cu_seqlens")
    M, U = scan_carry(k, v, g, beta, wy=wy, chunk_size=chunk_size, n_segments=n_segments,
                      seg_starts=seg_starts)
    h_in, _ = segment_compose(M, U, h0)
    return scan_emit(q, k, v, g, beta, h_in=h_in, wy=wy, chunk_size=chunk_size,
                     n_segments=n_segments, seg_starts=seg_starts,
                     output_final_state=output_final_state)
