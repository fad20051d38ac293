"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, run the oracle on the same values, and
measure the normwise error max|x - ref| / max|ref|."""
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
