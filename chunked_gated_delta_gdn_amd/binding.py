"""ctypes binding of ``libgdn.so`` (the C ABI in ``include/gdn.h``).

Argument marshalling only: every function here forwards plain integers and
device addresses to the entry point of the same name and turns a non-zero
status into an exception (``ValueError`` for invalid, unsupported or
out-of-order arguments and short workspaces, ``RuntimeError`` for launch
failures).  Nothing is
computed on the host and there is no fallback: if the library is missing the
first call raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same library (the sanitized host build of the CPU tests)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(PKG, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EORDER, GDN_ELAUNCH, GDN_EWORKSPACE = range(6)
GDN_F32, GDN_BF16 = 0, 1
GDN_SCAN_EMIT, GDN_SCAN_CARRY, GDN_SCAN_HEAD_EMIT_CARRY, GDN_SCAN_TAIL_EMIT = 0, 1, 2, 3
GDN_MAX_SEQS, GDN_MAX_SEGMENTS = 256, 64

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class GdnProblem(ctypes.Structure):
    """Mirror of ``gdn_problem`` in include/gdn.h."""
    _fields_ = [
        ("B", _i32), ("S", _i32), ("H", _i32), ("K", _i32), ("V", _i32), ("C", _i32),
        ("dtype", _i32), ("n_seqs", _i32),
        ("cu_seqlens", ctypes.POINTER(_i32)),
        ("n_segments", _i32),
        ("seg_starts", ctypes.POINTER(_i32)),
        ("max_piece_chunks", _i32),
        ("H_qk", _i32),
    ]


def make_problem(B, S, H, K, V, C, dtype, cu_seqlens=None, n_segments=1, seg_starts=None,
                 max_piece_chunks=0, H_qk=0):
    """Build a ``GdnProblem``; the host arrays it points to are kept alive on it."""
    p = GdnProblem()
    p.B, p.S, p.H, p.K, p.V, p.C, p.dtype = B, S, H, K, V, C, dtype
    p.n_segments = n_segments
    p.max_piece_chunks = max_piece_chunks
    p.H_qk = H_qk
    if cu_seqlens is not None:
        cu = [int(x) for x in cu_seqlens]
        arr = (_i32 * len(cu))(*cu)
        p._cu = arr
        p.n_seqs = len(cu) - 1
        p.cu_seqlens = ctypes.cast(arr, ctypes.POINTER(_i32))
    if seg_starts is not None:
        ss = [int(x) for x in seg_starts]
        arr = (_i32 * max(1, len(ss)))(*ss)
        p._ss = arr
        p.seg_starts = ctypes.cast(arr, ctypes.POINTER(_i32))
    return p


class GdnError(Exception):
    pass


class GdnValueError(GdnError, ValueError):
    pass


class GdnLaunchError(GdnError, RuntimeError):
    pass


_LIB = None


def library():
    """Load ``libgdn.so`` (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GdnProblem)
        sig = {
            "gdn_validate": (_i32, [P]),
            "gdn_num_pieces": (_i32, [P]),
            "gdn_wy_workspace_bytes": (ctypes.c_size_t, [P]),
            "gdn_segment_workspace_bytes": (ctypes.c_size_t, [P]),
            "gdn_chunk_prepare": (_i32, [P, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
            "gdn_scan": (_i32, [P, _i32] + [_vp] * 6 + [ctypes.c_size_t] + [_vp] * 6),
            "gdn_segment_compose": (_i32, [_i32] * 5 + [_vp] * 6),
            "gdn_piece_compose": (_i32, [P, _i32] + [_vp] * 6),
            "gdn_decode_step": (_i32, [_i32] * 6 + [_vp] * 8),
            "gdn_scan_backend": (_i32, [P]),
            "gdn_backward_workspace_bytes": (ctypes.c_size_t, [P]),
            "gdn_forward_workspace_bytes": (ctypes.c_size_t, [P]),
            "gdn_forward": (_i32, [P] + [_vp] * 9 + [ctypes.c_size_t, _vp]),
            "gdn_forward_noalloc": (_i32, [P] + [_vp] * 9),
            "gdn_backward": (_i32, [P] + [_vp] * 15 + [ctypes.c_size_t, _vp]),
            "gdn_causal_conv1d": (_i32, [_i32] * 6 + [ctypes.POINTER(_i32), _i32] + [_vp] * 6),
            "gdn_gated_rmsnorm": (_i32, [ctypes.c_int64, _i32, _i32, ctypes.c_float] + [_vp] * 5),
            "gdn_status_string": (ctypes.c_char_p, [_i32]),
            "gdn_last_error": (ctypes.c_char_p, []),
            "gdn_version": (_i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status, fn):
    if status == GDN_OK:
        return
    lib = library()
    msg = f"{fn}: {lib.gdn_status_string(status).decode()}: {lib.gdn_last_error().decode()}"
    if status == GDN_ELAUNCH:
        raise GdnLaunchError(msg)
    err = GdnValueError(msg)
    err.status = status
    raise err


def gdn_validate(problem, raise_on_error=True):
    st = library().gdn_validate(ctypes.byref(problem))
    if raise_on_error:
        _check(st, "gdn_validate")
    return st


def gdn_num_pieces(problem):
    """Pieces of a packed problem (segments B * R of a batch one); -1 if invalid."""
    return int(library().gdn_num_pieces(ctypes.byref(problem)))


def gdn_wy_workspace_bytes(problem):
    return int(library().gdn_wy_workspace_bytes(ctypes.byref(problem)))


def gdn_segment_workspace_bytes(problem):
    return int(library().gdn_segment_workspace_bytes(ctypes.byref(problem)))


def gdn_chunk_prepare(problem, k, v, g, beta, wy, wy_bytes, stream=0):
    _check(library().gdn_chunk_prepare(ctypes.byref(problem), k, v, g, beta, wy, wy_bytes, stream),
           "gdn_chunk_prepare")


def gdn_scan(problem, mode, q, k, v, g, beta, wy, wy_bytes, h_in, o, h_out, M_out, U_out, stream=0):
    _check(library().gdn_scan(ctypes.byref(problem), mode, q, k, v, g, beta, wy, wy_bytes, h_in, o, h_out,
                              M_out, U_out, stream), "gdn_scan")


def gdn_forward_workspace_bytes(problem):
    return int(library().gdn_forward_workspace_bytes(ctypes.byref(problem)))


def gdn_forward(problem, q, k, v, g, beta, h0, o, h_out, workspace, workspace_bytes, stream=0):
    _check(library().gdn_forward(ctypes.byref(problem), q, k, v, g, beta, h0, o, h_out, workspace,
                                 workspace_bytes, stream), "gdn_forward")


def gdn_forward_noalloc(problem, q, k, v, g, beta, h0, o, h_out, stream=0):
    _check(library().gdn_forward_noalloc(ctypes.byref(problem), q, k, v, g, beta, h0, o, h_out, stream),
           "gdn_forward_noalloc")


GDN_FORWARD_SCRATCH_BYTES = 64 << 20


def gdn_segment_compose(R, N, H, K, V, M, U, h0, h_in, h_final, stream=0):
    _check(library().gdn_segment_compose(R, N, H, K, V, M, U, h0, h_in, h_final, stream),
           "gdn_segment_compose")


def gdn_piece_compose(problem, first, M, U, h_seed, h_in, h_final, stream=0):
    _check(library().gdn_piece_compose(ctypes.byref(problem), first, M, U, h_seed, h_in, h_final, stream),
           "gdn_piece_compose")


def gdn_decode_step(B, H, H_qk, K, V, dtype, q, k, v, g, beta, state, o, stream=0):
    _check(library().gdn_decode_step(B, H, H_qk, K, V, dtype, q, k, v, g, beta, state, o, stream),
           "gdn_decode_step")


def gdn_causal_conv1d(B, S, D, W, dtype, activation, cu_seqlens, x, weight, state_in, state_out, y, stream=0):
    """cu_seqlens: a host sequence of n_seqs + 1 offsets, or None (batch mode)."""
    if cu_seqlens is None:
        cu, n = None, 0
    else:
        vals = [int(c) for c in cu_seqlens]
        cu, n = (_i32 * len(vals))(*vals), len(vals) - 1
    _check(library().gdn_causal_conv1d(B, S, D, W, dtype, activation,
                                       ctypes.cast(cu, ctypes.POINTER(_i32)) if cu is not None else None, n,
                                       x, weight, state_in, state_out, y, stream), "gdn_causal_conv1d")


def gdn_gated_rmsnorm(rows, V, dtype, eps, o, z, weight, y, stream=0):
    _check(library().gdn_gated_rmsnorm(rows, V, dtype, eps, o, z, weight, y, stream), "gdn_gated_rmsnorm")


def gdn_backward_workspace_bytes(problem):
    return int(library().gdn_backward_workspace_bytes(ctypes.byref(problem)))


def gdn_backward(problem, q, k, v, g, beta, h0, dout, dhT, dq, dk, dv, dg, dbeta, dh0,
                 workspace, workspace_bytes, stream=0):
    _check(library().gdn_backward(ctypes.byref(problem), q, k, v, g, beta, h0, dout, dhT, dq, dk,
                                  dv, dg, dbeta, dh0, workspace, workspace_bytes, stream),
           "gdn_backward")


def gdn_scan_backend(problem):
    """1 if gdn_scan runs on the matrix cores for this problem, 0 on the vector ALU."""
    return int(library().gdn_scan_backend(ctypes.byref(problem)))


def gdn_version():
    return int(library().gdn_version())
