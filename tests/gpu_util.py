"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, run the oracle on the same values, and
measure the normwise error max|x - ref| / max|ref|, over a whole tensor and
over its worst (sequence, head) slice."""
import sys

import numpy as np
import torch

import oracle
import chunked_gated_delta_gdn_amd as gdn

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}   # bound on normwise relative error vs the fp64 oracle


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def tdt(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def device_inputs(x):
    dt = tdt(x.dtype)
    return dict(q=to_dev(x.q, dt), k=to_dev(x.k, dt), v=to_dev(x.v, dt), g=to_dev(x.g),
                beta=to_dev(x.beta), h0=None if x.h0 is None else to_dev(x.h0))


def run_forward(x, n_segments=1, seg_starts=None, reuse_wy=False, h0=True, schedule="auto",
                max_piece_chunks=None):
    d = device_inputs(x)
    o, hT = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"] if h0 else None,
                        chunk_size=x.C, cu_seqlens=x.cu_seqlens, n_segments=n_segments,
                        seg_starts=seg_starts, reuse_wy=reuse_wy, schedule=schedule,
                        max_piece_chunks=max_piece_chunks)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), hT.cpu().numpy()


def oracle_forward(x, heads=None, h0=True):
    """fp64 oracle on the same (dtype-rounded) values, optionally on a subset of heads."""
    hs = slice(None) if heads is None else list(heads)
    h0a = x.h0[:, hs] if (h0 and x.h0 is not None) else None
    if x.cu_seqlens is not None:
        return oracle.forward_packed(x.cu_seqlens, x.q[0][:, hs], x.k[0][:, hs], x.v[0][:, hs],
                                     x.g[0][:, hs], x.beta[0][:, hs], h0=h0a)
    return oracle.forward(x.q[:, :, hs], x.k[:, :, hs], x.v[:, :, hs], x.g[:, :, hs],
                          x.beta[:, :, hs], h0=h0a)


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    return float(num / den) if den > 0 else float(num)


def slice_err(x, ref, axes):
    """Worst normwise error over the slices that fix the given axes (e.g. the
    (b, h) slices of o [B,S,H,V] for axes (0, 2)): a fault confined to one
    head or one sequence is not diluted by the magnitude of the others."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rest = [a for a in range(ref.ndim) if a not in axes]
    xs = np.transpose(x, list(axes) + rest).reshape(-1, int(np.prod([ref.shape[a] for a in rest])))
    rs = np.transpose(ref, list(axes) + rest).reshape(xs.shape)
    num = np.max(np.abs(xs - rs), axis=1)
    den = np.max(np.abs(rs), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def o_axes(o):
    """Slice axes of an output tensor: (b, h) of [B,S,H,V], h of packed [T,H,V]."""
    return (0, 2) if np.ndim(o) == 4 else (1,)


def check_forward(x, o, hT, o_ref, h_ref, tol=None, what=""):
    """Outputs and final states against the oracle: the normwise error of each
    tensor and of its worst (sequence, head) slice, both within tol."""
    tol = TOL[x.dtype] if tol is None else tol
    eo, eh = rel_err(o, o_ref), rel_err(hT, h_ref)
    so, sh = slice_err(o, o_ref, o_axes(o_ref)), slice_err(hT, h_ref, (0, 1))
    cu = getattr(x, "cu_seqlens", None)
    if cu is not None and np.ndim(o_ref) == 3 and len(o_ref) == int(cu[-1]):
        # packed [T,H,V]: every (sequence, head) slice on its own
        for n in range(len(cu) - 1):
            a, b = int(cu[n]), int(cu[n + 1])
            if b > a:
                so = max(so, slice_err(np.asarray(o)[a:b], o_ref[a:b], (1,)))
    say(f"  {x.name} {what}: err(o)={eo:.3e} (worst head {so:.3e}) err(hT)={eh:.3e} "
        f"(worst head {sh:.3e}) tol={tol:g}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= tol, f"output error {eo} > {tol}"
    assert eh <= tol, f"final state error {eh} > {tol}"
    assert so <= tol, f"worst (sequence, head) output error {so} > {tol}"
    assert sh <= tol, f"worst (sequence, head) final state error {sh} > {tol}"
    return max(eo, eh, so, sh)
