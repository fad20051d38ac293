"""Tensor-level calls of the library (PyTorch supplies device memory and streams).

Each function checks shapes and dtypes, allocates the outputs with torch and
forwards device addresses to the C entry point of the same name.  ``forward``
chains the entry points exactly as the three-phase pass of the MaxText PR "Add
context parallelism to the Gated Delta Net" (section "Implementation")
describes: one segment runs a single emitting scan; several segments run the
carrying scan (phase 1), the exclusive segment scan (phase 2) and the emitting
scan from the true incoming states (phase 3).  Packed batches run the same
pass over pieces of their long sequences (``forward_packed``).
"""
import functools
import heapq

import torch

from . import binding as _b

__all__ = ["problem_for", "chunk_prepare", "scan_emit", "scan_carry", "segment_compose",
           "segment_bounds", "forward_segmented", "num_pieces", "scan_tail_emit", "piece_compose",
           "plan_pieces", "forward_packed", "decode_step", "forward", "causal_conv1d", "gated_rmsnorm",
           "backward", "chunk_gated_delta_rule"]


def _dtype_code(t):
    if t.dtype == torch.float32:
        return _b.GDN_F32
    if t.dtype == torch.bfloat16:
        return _b.GDN_BF16
    raise ValueError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _addr(t):
    return None if t is None else t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


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


def problem_for(k, v, chunk_size, cu_seqlens=None, n_segments=1, seg_starts=None, max_piece_chunks=0):
    """The ``gdn_problem`` of batch tensors k [B,S,H_qk,K], v [B,S,H,V] (H_qk
    key heads for H value heads, H a multiple of H_qk)."""
    B, S, Hk, K = k.shape
    H, V = v.shape[2], v.shape[3]
    return _b.make_problem(B, S, H, K, V, chunk_size, _dtype_code(k), cu_seqlens=cu_seqlens,
                           n_segments=n_segments, seg_starts=seg_starts,
                           max_piece_chunks=max_piece_chunks, H_qk=0 if Hk == H else Hk)


def num_pieces(k, v, chunk_size, cu_seqlens, max_piece_chunks):
    """Pieces P of a packed problem (``gdn_num_pieces``)."""
    p = problem_for(k, v, chunk_size, cu_seqlens, max_piece_chunks=max_piece_chunks)
    _b.gdn_validate(p)
    return _b.gdn_num_pieces(p)


def _n_seqs(k, cu_seqlens):
    return k.shape[0] if cu_seqlens is None else len(cu_seqlens) - 1


def _check_inputs(q, k, v, g, beta):
    """Shapes q, k [B,S,H_qk,K]; v [B,S,H,V]; g, beta [B,S,H] (H a multiple of
    H_qk: value head h reads key head h // (H // H_qk)).  Returns B, S, H, K, V
    with H the value (state) heads."""
    dev = k.device
    B, S, Hk, K = k.shape
    if v.dim() != 4 or v.shape[:2] != k.shape[:2]:
        raise ValueError(f"v has shape {tuple(v.shape)}, expected [B,S,H,V] with B,S of k {tuple(k.shape)}")
    H, V = v.shape[2], v.shape[3]
    if Hk < 1 or H % Hk != 0:
        raise ValueError(f"value heads {H} are not a multiple of key heads {Hk}")
    if q is not None:
        _need(q, "q", (B, S, Hk, K), k.dtype, dev)
    _need(k, "k", (B, S, Hk, K), k.dtype, dev)
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
    _b.gdn_chunk_prepare(p, _addr(k), _addr(v), _addr(g), _addr(beta), _addr(wy), _nbytes(wy),
                         _stream(k.device))
    return wy


def split_wy(wy, k, v, chunk_size, cu_seqlens=None):
    """Views (w [n_chunks,H,C,K], u [n_chunks,H,C,V]) of a WY workspace (H value heads)."""
    H, K, V = v.shape[2], k.shape[3], v.shape[3]
    n_chunks = wy.numel() // (H * chunk_size * (K + V))
    w = wy[: n_chunks * H * chunk_size * K].view(n_chunks, H, chunk_size, K)
    u = wy[n_chunks * H * chunk_size * K:].view(n_chunks, H, chunk_size, V)
    return w, u


def scan_emit(q, k, v, g, beta, h_in=None, wy=None, chunk_size=64, cu_seqlens=None,
              n_segments=1, seg_starts=None, output_final_state=True, out=None, max_piece_chunks=0):
    """Emitting scan (``gdn_scan`` with GDN_SCAN_EMIT): returns (o, h_out).

    h_in is [N,H,K,V] for one segment, or [R,N,H,K,V] (the state entering each
    segment) for R segments, or [P,H,K,V] (per piece) for a packed problem cut
    into pieces; None means zero state everywhere."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    N = _n_seqs(k, cu_seqlens)
    p = problem_for(k, v, chunk_size, cu_seqlens, n_segments, seg_starts, max_piece_chunks)
    _b.gdn_validate(p)
    if h_in is not None:
        if cu_seqlens is not None:
            shape = (_b.gdn_num_pieces(p), H, K, V)
        else:
            shape = (N, H, K, V) if n_segments == 1 else (n_segments, N, H, K, V)
        _need(h_in, "h_in", shape, torch.float32, dev)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    o = out if out is not None else torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, S, H, V), k.dtype, dev)
    h_out = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    _b.gdn_scan(p, _b.GDN_SCAN_EMIT, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), _nbytes(wy), _addr(h_in), _addr(o), _addr(h_out), None, None, _stream(dev))
    return o, h_out


def scan_head_carry(q, k, v, g, beta, h_in=None, wy=None, chunk_size=64, n_segments=2, seg_starts=None,
                    out=None, cu_seqlens=None, max_piece_chunks=0, h_out=None):
    """Segment 0 emitted, segments 1 .. R-1 carried (``gdn_scan`` with
    GDN_SCAN_HEAD_EMIT_CARRY): returns (o, h1, M [R-1,B,H,K,K], U [R-1,B,H,K,V]).
    o holds segment 0's outputs (other tokens untouched when ``out`` is given),
    h1 [B,H,K,V] is segment 0's final state, the state entering segment 1.

    Packed problems (cu_seqlens, max_piece_chunks): the first piece of every
    sequence is emitted from h_in [N,H,K,V] and the middle pieces carried;
    returns (o, h1 [N,H,K,V], M [P,H,K,K], U [P,H,K,V]) with the rows of
    pieces that are not carried left unwritten."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    packed = cu_seqlens is not None
    N = _n_seqs(k, cu_seqlens)
    p = problem_for(k, v, chunk_size, cu_seqlens, 1 if packed else n_segments, None if packed else seg_starts,
                    max_piece_chunks)
    _b.gdn_validate(p)
    if h_in is not None:
        _need(h_in, "h_in", (N, H, K, V), torch.float32, dev)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    o = out if out is not None else torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, S, H, V), k.dtype, dev)
    h1 = h_out if h_out is not None else torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    _need(h1, "h_out", (N, H, K, V), torch.float32, dev)
    lead = (_b.gdn_num_pieces(p),) if packed else (n_segments - 1, B)
    M = torch.empty(lead + (H, K, K), dtype=torch.float32, device=dev)
    U = torch.empty(lead + (H, K, V), dtype=torch.float32, device=dev)
    _b.gdn_scan(p, _b.GDN_SCAN_HEAD_EMIT_CARRY, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), _nbytes(wy), _addr(h_in), _addr(o), _addr(h1), _addr(M), _addr(U), _stream(dev))
    return o, h1, M, U


def scan_carry(k, v, g, beta, wy=None, chunk_size=64, n_segments=1, seg_starts=None, cu_seqlens=None,
               max_piece_chunks=0):
    """Carrying zero-state scan (``gdn_scan`` with GDN_SCAN_CARRY): returns
    (M [R,B,H,K,K], U [R,B,H,K,V]) with h_end = M h_start + U per segment, or
    (M [P,H,K,K], U [P,H,K,V]) per piece of a packed problem."""
    B, S, H, K, V = _check_inputs(None, k, v, g, beta)
    dev = k.device
    p = problem_for(k, v, chunk_size, cu_seqlens, n_segments, seg_starts, max_piece_chunks)
    _b.gdn_validate(p)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    lead = (_b.gdn_num_pieces(p),) if cu_seqlens is not None else (n_segments, B)
    M = torch.empty(lead + (H, K, K), dtype=torch.float32, device=dev)
    U = torch.empty(lead + (H, K, V), dtype=torch.float32, device=dev)
    _b.gdn_scan(p, _b.GDN_SCAN_CARRY, None, _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), _nbytes(wy), None, None, None, _addr(M), _addr(U), _stream(dev))
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


def scan_tail_emit(q, k, v, g, beta, h_in, cu_seqlens, max_piece_chunks, wy=None, chunk_size=64,
                   out=None, h_out=None):
    """Pieces 1 .. R_n-1 of every sequence of a packed problem emitted from
    h_in [P,H,K,V] (``gdn_scan`` with GDN_SCAN_TAIL_EMIT): returns (o, h_out).
    Tokens of first pieces in o, and h_out rows of one-piece sequences, are not
    written (pass ``out`` / ``h_out`` holding them)."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    N = _n_seqs(k, cu_seqlens)
    p = problem_for(k, v, chunk_size, cu_seqlens, max_piece_chunks=max_piece_chunks)
    _b.gdn_validate(p)
    if h_in is not None:
        _need(h_in, "h_in", (_b.gdn_num_pieces(p), H, K, V), torch.float32, dev)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    o = out if out is not None else torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, S, H, V), k.dtype, dev)
    if h_out is None:
        h_out = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    _need(h_out, "h_out", (N, H, K, V), torch.float32, dev)
    _b.gdn_scan(p, _b.GDN_SCAN_TAIL_EMIT, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta),
                _addr(wy), _nbytes(wy), _addr(h_in), _addr(o), _addr(h_out), None, None, _stream(dev))
    return o, h_out


def piece_compose(k, v, M, U, cu_seqlens, max_piece_chunks, chunk_size=64, first=0, h_seed=None,
                  want_final=False):
    """Per-sequence scan over the pieces of a packed problem
    (``gdn_piece_compose``): returns (h_in [P,H,K,V], h_final [N,H,K,V] or None).
    Rows of h_in before piece ``first`` of each sequence are not written."""
    K = k.shape[3]
    H, V = v.shape[2], v.shape[3]
    dev = M.device
    N = _n_seqs(k, cu_seqlens)
    p = problem_for(k, v, chunk_size, cu_seqlens, max_piece_chunks=max_piece_chunks)
    _b.gdn_validate(p)
    P = _b.gdn_num_pieces(p)
    _need(M, "M", (P, H, K, K), torch.float32, dev)
    _need(U, "U", (P, H, K, V), torch.float32, dev)
    if h_seed is not None:
        _need(h_seed, "h_seed", (N, H, K, V), torch.float32, dev)
    h_in = torch.empty((P, H, K, V), dtype=torch.float32, device=dev)
    h_final = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if want_final else None
    _b.gdn_piece_compose(p, first, _addr(M), _addr(U), _addr(h_seed), _addr(h_in), _addr(h_final),
                         _stream(dev))
    return h_in, h_final


def _lpt_makespan(items, n_cu):
    """Finish time of list scheduling (longest first) of `items` = [(length,
    count)] workgroups on n_cu compute units, one workgroup per unit."""
    free = [0] * n_cu
    for length, count in sorted(items, reverse=True):
        if length == 0:
            continue
        for _ in range(count):
            heapq.heapreplace(free, free[0] + length)
    return max(free)


def _piece_chunks(nc, m):
    """Chunk counts of the pieces of a sequence of nc chunks (the library's split)."""
    if m <= 0 or nc <= m:
        return [nc]
    R = -(-nc // m)
    return [(s + 1) * nc // R - s * nc // R for s in range(R)]


@functools.lru_cache(maxsize=256)
def plan_pieces(chunks, heads, n_cu, overhead=12, max_pieces=_b.GDN_MAX_SEQS):
    """max_piece_chunks for a packed batch whose sequences have ``chunks``
    chunks (a tuple), or 0 when cutting pieces does not pay.

    Cost model: every (piece, head) runs as two workgroups, one per compute
    unit, for as many chunk steps as the piece has chunks; the emitting and
    carrying steps cost about the same; a launch takes the longest-first list
    schedule's makespan.  One piece per sequence is one launch; pieces take
    two launches (first pieces emitted with the middle ones carried; then the
    rest emitted) plus ``overhead`` chunk steps for the compose and the extra
    launch.  Candidates are the caps that split the longest sequence into
    2 .. 32 pieces."""
    w = 2 * heads
    best, best_cost = 0, _lpt_makespan([(c, w) for c in chunks], n_cu)
    top = max(chunks, default=0)
    for r in range(2, 33):
        m = -(-top // r)
        if m < 1:
            break
        first, tail = [], []
        n_pieces = 0
        for c in chunks:
            pcs = _piece_chunks(c, m)
            n_pieces += len(pcs)
            first.append((pcs[0], w))
            first += [(x, w) for x in pcs[1:-1]]
            tail += [(x, w) for x in pcs[1:]]
        if n_pieces > max_pieces:
            break
        cost = _lpt_makespan(first, n_cu) + _lpt_makespan(tail, n_cu) + overhead
        if cost < best_cost:
            best, best_cost = m, cost
    return best


def forward_packed(q, k, v, g, beta, cu_seqlens, h0=None, chunk_size=64, max_piece_chunks=None,
                   wy=None, output_final_state=True, timer=None):
    """Packed batch with long sequences cut into pieces: the segment pass
    without redundant work over pieces (first pieces emitted beside the
    carried middle ones, the per-sequence scan from the first pieces' final
    states, then the other pieces emitted).  ``max_piece_chunks=None`` picks
    the cut with ``plan_pieces``; a cut that leaves every sequence whole runs
    one emitting scan.  Returns (o, final states or None).

    One problem description, one validation and two allocations serve the
    three launches, so that short workloads are not bound by host work."""
    timer = timer or _untimed
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    if max_piece_chunks is None:
        chunks = tuple(-(-(cu[n + 1] - cu[n]) // chunk_size) for n in range(N))
        max_piece_chunks = plan_pieces(chunks, H, _n_cu(dev))
    p = problem_for(k, v, chunk_size, cu, max_piece_chunks=max_piece_chunks)
    _b.gdn_validate(p)
    P = _b.gdn_num_pieces(p)
    if h0 is not None:
        _need(h0, "h0", (N, H, K, V), torch.float32, dev)
    if wy is not None:
        _need(wy, "wy", (_b.gdn_wy_workspace_bytes(p) // k.element_size(),), k.dtype, dev)
    st = _stream(dev)
    args = (_addr(q), _addr(k), _addr(v), _addr(g), _addr(beta), _addr(wy), _nbytes(wy))
    o = torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    if P == N:
        hT = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if output_final_state else None
        timer("scan_emit", lambda: _b.gdn_scan(p, _b.GDN_SCAN_EMIT, *args, _addr(h0), _addr(o), _addr(hT),
                                               None, None, st))
        return o, hT
    # one fp32 buffer: M [P,H,K,K], U [P,H,K,V], h_in [P,H,K,V], final states [N,H,K,V]
    nm, ns = P * H * K * K, P * H * K * V
    buf = torch.empty(nm + 2 * ns + N * H * K * V, dtype=torch.float32, device=dev)
    M, U, h_in, hT = buf[:nm], buf[nm:nm + ns], buf[nm + ns:nm + 2 * ns], buf[nm + 2 * ns:]
    timer("scan_head_carry", lambda: _b.gdn_scan(p, _b.GDN_SCAN_HEAD_EMIT_CARRY, *args, _addr(h0), _addr(o),
                                                 _addr(hT), _addr(M), _addr(U), st))
    timer("piece_compose", lambda: _b.gdn_piece_compose(p, 1, _addr(M), _addr(U), _addr(hT), _addr(h_in), None,
                                                        st))
    timer("scan_tail_emit", lambda: _b.gdn_scan(p, _b.GDN_SCAN_TAIL_EMIT, *args, _addr(h_in), _addr(o),
                                                _addr(hT), None, None, st))
    return o, (hT.view(N, H, K, V) if output_final_state else None)


@functools.lru_cache(maxsize=16)
def _n_cu_of(index):
    return torch.cuda.get_device_properties(index).multi_processor_count


def _n_cu(dev):
    return _n_cu_of(dev.index if dev.index is not None else torch.cuda.current_device())


def decode_step(q, k, v, g, beta, state, out=None):
    """One recurrent step (``gdn_decode_step``), updating ``state`` in place.

    q, k [B,H_qk,K]; v [B,H,V]; g, beta [B,H] fp32; state [B,H,K,V] fp32 (H a
    multiple of H_qk).  Returns o [B,H,V]."""
    B, Hk, K = k.shape
    H, V = v.shape[1], v.shape[2]
    dev = k.device
    if Hk < 1 or H % Hk != 0:
        raise ValueError(f"value heads {H} are not a multiple of key heads {Hk}")
    _need(q, "q", (B, Hk, K), k.dtype, dev)
    _need(v, "v", (B, H, V), k.dtype, dev)
    _need(g, "g", (B, H), torch.float32, dev)
    _need(beta, "beta", (B, H), torch.float32, dev)
    _need(state, "state", (B, H, K, V), torch.float32, dev)
    o = out if out is not None else torch.empty((B, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, H, V), k.dtype, dev)
    _b.gdn_decode_step(B, H, Hk, K, V, _dtype_code(k), _addr(q), _addr(k), _addr(v), _addr(g),
                       _addr(beta), _addr(state), _addr(o), _stream(dev))
    return o


def causal_conv1d(x, weight, state=None, cu_seqlens=None, activation="silu", want_state=True, state_out=None):
    """Depthwise causal convolution before the core (``gdn_causal_conv1d``).

    x [B,S,D] (or [1,T,D] with cu_seqlens), weight [D,W], state [N,D,W-1] or
    None (zeros), all in x's dtype.  Returns (y like x, the state after each
    sequence [N,D,W-1] or None).  ``state_out`` may be ``state`` itself for
    one-token steps (decode)."""
    dev = x.device
    B, S, D = x.shape
    W = weight.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    _need(x, "x", (B, S, D), x.dtype, dev)
    _need(weight, "weight", (D, W), x.dtype, dev)
    if state is not None:
        _need(state, "state", (N, D, W - 1), x.dtype, dev)
    if state_out is None and want_state:
        state_out = torch.empty((N, D, W - 1), dtype=x.dtype, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", (N, D, W - 1), x.dtype, dev)
    act = {"silu": 1, "none": 0, None: 0}[activation]
    y = torch.empty_like(x)
    _b.gdn_causal_conv1d(B, S, D, W, _dtype_code(x), act, cu_seqlens, _addr(x), _addr(weight), _addr(state),
                         _addr(state_out), _addr(y), _stream(dev))
    return y, state_out


def gated_rmsnorm(o, weight, z=None, eps=1e-6, out=None):
    """Gated RMSNorm after the core (``gdn_gated_rmsnorm``): each vector of the
    last axis of o (V elements) becomes o / sqrt(mean(o^2) + eps) * weight *
    SiLU(z).  weight [V] fp32; z like o or None; ``out`` may be o."""
    dev = o.device
    V = o.shape[-1]
    _need(o, "o", tuple(o.shape), o.dtype, dev)
    _need(weight, "weight", (V,), torch.float32, dev)
    if z is not None:
        _need(z, "z", tuple(o.shape), o.dtype, dev)
    y = out if out is not None else torch.empty_like(o)
    _need(y, "out", tuple(o.shape), o.dtype, dev)
    _b.gdn_gated_rmsnorm(o.numel() // V, V, _dtype_code(o), float(eps), _addr(o), _addr(z), _addr(weight),
                         _addr(y), _stream(dev))
    return y


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


def forward_fused(q, k, v, g, beta, h0=None, chunk_size=64, cu_seqlens=None, n_segments=1, seg_starts=None,
                  max_piece_chunks=None, output_final_state=True, out=None, h_out=None, workspace=None):
    """The whole forward in one library call (``gdn_forward``): one emitting
    scan per sequence, the segment pass (batch, n_segments > 1) or the piece
    schedule (packed; max_piece_chunks None = ``plan_pieces``).  Returns (o,
    final state or None).  ``workspace`` (uint8, at least
    gdn_forward_workspace_bytes) is allocated when not given."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    N = _n_seqs(k, cu_seqlens)
    if cu_seqlens is not None:
        cu = [int(x) for x in cu_seqlens]
        if max_piece_chunks is None:
            chunks = tuple(-(-(cu[n + 1] - cu[n]) // chunk_size) for n in range(N))
            max_piece_chunks = plan_pieces(chunks, H, _n_cu(dev))
    else:
        cu = None
        max_piece_chunks = 0
    p = problem_for(k, v, chunk_size, cu, n_segments, seg_starts, max_piece_chunks)
    _b.gdn_validate(p)
    if h0 is not None:
        _need(h0, "h0", (N, H, K, V), torch.float32, dev)
    o = out if out is not None else torch.empty((B, S, H, V), dtype=k.dtype, device=dev)
    _need(o, "o", (B, S, H, V), k.dtype, dev)
    if h_out is None and output_final_state:
        h_out = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    if h_out is not None:
        _need(h_out, "h_out", (N, H, K, V), torch.float32, dev)
    need = _b.gdn_forward_workspace_bytes(p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _b.gdn_forward(p, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta), _addr(h0), _addr(o), _addr(h_out),
                   _addr(workspace), _nbytes(workspace), _stream(dev))
    return o, h_out


def forward(q, k, v, g, beta, h0=None, chunk_size=64, cu_seqlens=None, n_segments=1,
            seg_starts=None, reuse_wy=False, output_final_state=True, schedule="auto",
            max_piece_chunks=None):
    """Chunked gated delta rule forward: returns (o, final state or None).

    n_segments > 1 runs the three-phase segment pass; reuse_wy prepares the WY
    factors once (``gdn_chunk_prepare``) and hands them to both scans instead of
    recomputing them inside each scan.  schedule="auto" with recomputed WY
    factors is one ``gdn_forward`` call (``forward_fused``: the segment pass
    without its redundant work); "plain" always runs the full carrying pass
    over every segment.

    Packed batches (cu_seqlens) take max_piece_chunks instead of segments:
    None or "auto" lets schedule="auto" choose the cut (``plan_pieces``; no cut
    when the WY factors are reused or the schedule is "plain"), 0 keeps every
    sequence whole; "auto" runs ``gdn_forward`` (``forward_packed`` with reused
    WY factors), "plain" the carrying pass
    over every piece, ``gdn_piece_compose`` from the initial states, and the
    emitting pass over every piece.  A batch [B,S,H,*] given max_piece_chunks
    ("auto" or a number) runs as the packed batch of its B sequences."""
    if schedule not in ("auto", "plain"):
        raise ValueError(f"unknown schedule {schedule!r}")
    if cu_seqlens is None and max_piece_chunks is not None:
        if n_segments != 1:
            raise ValueError("pieces replace segments: pass n_segments=1 with max_piece_chunks")
        B, S, H = v.shape[:3]
        flat = lambda t: t.reshape((1, B * S) + tuple(t.shape[2:]))
        o, hT = forward(flat(q), flat(k), flat(v), flat(g), flat(beta), h0=h0, chunk_size=chunk_size,
                        cu_seqlens=[b * S for b in range(B + 1)], reuse_wy=reuse_wy,
                        output_final_state=output_final_state, schedule=schedule,
                        max_piece_chunks=max_piece_chunks)
        return o.view(B, S, H, v.shape[-1]), hT
    if max_piece_chunks == "auto":
        max_piece_chunks = None
    if cu_seqlens is not None:
        if n_segments != 1:
            raise ValueError("packed batches take max_piece_chunks, not segments")
        wy = chunk_prepare(k, v, g, beta, chunk_size, cu_seqlens) if reuse_wy else None
        if schedule == "auto":
            m = max_piece_chunks if max_piece_chunks is not None else (0 if reuse_wy else None)
            if wy is None:
                return forward_fused(q, k, v, g, beta, h0=h0, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                                     max_piece_chunks=m, output_final_state=output_final_state)
            return forward_packed(q, k, v, g, beta, cu_seqlens, h0=h0, chunk_size=chunk_size,
                                  max_piece_chunks=m, wy=wy, output_final_state=output_final_state)
        m = max_piece_chunks or 0
        if m == 0:
            return scan_emit(q, k, v, g, beta, h_in=h0, wy=wy, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                             output_final_state=output_final_state)
        M, U = scan_carry(k, v, g, beta, wy=wy, chunk_size=chunk_size, cu_seqlens=cu_seqlens, max_piece_chunks=m)
        h_in, _ = piece_compose(k, v, M, U, cu_seqlens, m, chunk_size, first=0, h_seed=h0)
        return scan_emit(q, k, v, g, beta, h_in=h_in, wy=wy, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                         output_final_state=output_final_state, max_piece_chunks=m)
    if schedule == "auto" and not reuse_wy:
        return forward_fused(q, k, v, g, beta, h0=h0, chunk_size=chunk_size, n_segments=n_segments,
                             seg_starts=seg_starts, output_final_state=output_final_state)
    wy = chunk_prepare(k, v, g, beta, chunk_size, cu_seqlens) if reuse_wy else None
    if n_segments == 1:
        return scan_emit(q, k, v, g, beta, h_in=h0, wy=wy, chunk_size=chunk_size,
                         cu_seqlens=cu_seqlens, output_final_state=output_final_state)
    M, U = scan_carry(k, v, g, beta, wy=wy, chunk_size=chunk_size, n_segments=n_segments,
                      seg_starts=seg_starts)
    h_in, _ = segment_compose(M, U, h0)
    return scan_emit(q, k, v, g, beta, h_in=h_in, wy=wy, chunk_size=chunk_size,
                     n_segments=n_segments, seg_starts=seg_starts,
                     output_final_state=output_final_state)


def backward(q, k, v, g, beta, do, h0=None, dhT=None, chunk_size=64, cu_seqlens=None, want_dh0=True,
             n_segments=1, seg_starts=None, max_piece_chunks=0):
    """Gradients through the forward pass (``gdn_backward``).

    q, k [B,S,H_qk,K]; v, do [B,S,H,V] (fp32 or bf16); g, beta [B,S,H] fp32;
    h0, dhT [N,H,K,V] fp32 or None (zero).  Packed batches pass B == 1 and
    cu_seqlens.  n_segments / seg_starts (batch) and max_piece_chunks
    (packed) cut each sequence into parts whose state scans run in parallel,
    as in ``forward``.  Returns (dq, dk, dv, dg, dbeta, dh0 or None), each in
    the layout and dtype of its input (dh0 fp32)."""
    B, S, H, K, V = _check_inputs(q, k, v, g, beta)
    dev = k.device
    N = _n_seqs(k, cu_seqlens)
    _need(do, "do", (B, S, H, V), k.dtype, dev)
    if h0 is not None:
        _need(h0, "h0", (N, H, K, V), torch.float32, dev)
    if dhT is not None:
        _need(dhT, "dhT", (N, H, K, V), torch.float32, dev)
    p = problem_for(k, v, chunk_size, cu_seqlens, n_segments=n_segments, seg_starts=seg_starts,
                    max_piece_chunks=max_piece_chunks or 0)
    _b.gdn_validate(p)
    nbytes = _b.gdn_backward_workspace_bytes(p)
    ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    dh0 = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if want_dh0 else None
    _b.gdn_backward(p, _addr(q), _addr(k), _addr(v), _addr(g), _addr(beta), _addr(h0), _addr(do),
                    _addr(dhT), _addr(dq), _addr(dk), _addr(dv), _addr(dg), _addr(dbeta), _addr(dh0),
                    _addr(ws), nbytes, _stream(dev))
    return dq, dk, dv, dg, dbeta, dh0


class _ChunkGatedDeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, h0, chunk_size, cu_seqlens, n_segments, max_piece_chunks):
        o, hT = forward(q, k, v, g, beta, h0=h0, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                        n_segments=n_segments, max_piece_chunks=max_piece_chunks)
        ctx.save_for_backward(q, k, v, g, beta, h0)
        ctx.chunk_size, ctx.cu_seqlens = chunk_size, cu_seqlens
        # the backward's state scans take the same cut (an automatic piece plan
        # is the forward's choice, so the backward keeps whole sequences)
        ctx.n_segments = n_segments if cu_seqlens is None else 1
        ctx.max_piece_chunks = max_piece_chunks if isinstance(max_piece_chunks, int) else 0
        return o, hT

    @staticmethod
    def backward(ctx, do, dhT):
        q, k, v, g, beta, h0 = ctx.saved_tensors
        dq, dk, dv, dg, dbeta, dh0 = backward(
            q, k, v, g, beta, do.contiguous(), h0=h0,
            dhT=None if dhT is None else dhT.contiguous(), chunk_size=ctx.chunk_size,
            cu_seqlens=ctx.cu_seqlens, want_dh0=h0 is not None and ctx.needs_input_grad[5],
            n_segments=ctx.n_segments, max_piece_chunks=ctx.max_piece_chunks)
        return dq, dk, dv, dg, dbeta, dh0, None, None, None, None


def chunk_gated_delta_rule(q, k, v, g, beta, h0=None, chunk_size=64, cu_seqlens=None, n_segments=1,
                           max_piece_chunks=None):
    """Differentiable forward: (o, final state), with ``backward`` as its
    gradient (torch.autograd).  Shapes and the forward's schedule (segments;
    packed batches cut into pieces of at most max_piece_chunks chunks, None =
    planned) as ``forward``; q, k may have fewer heads than v (grouped key
    heads)."""
    return _ChunkGatedDeltaRule.apply(q, k, v, g, beta, h0, chunk_size, cu_seqlens, n_segments,
                                      max_piece_chunks)
