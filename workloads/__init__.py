"""Seeded synthetic inputs for the gated delta rule forward pass.

Shared by the tests, the benchmark and the smoke check; used by both the HIP
path and the CPU oracle.  This module holds none of the method's arithmetic:
only random draws, the input transforms of the workload recipe (L2
normalisation of q and k, sigmoid for beta, negative softplus for the
log-decay g) and round-to-nearest-even to bfloat16.

Recipe (one ``numpy.random.default_rng(seed)`` per workload; every draw fp32):
  lengths (packed workloads only) -> q, k, v ~ N(0,1) -> beta logits ~ N(0,1)
  -> g logits ~ N(0,1) -> initial state ~ N(0, std^2).
  q, k are L2-normalised over the head dimension, beta = sigmoid(logit),
  g = -softplus(logit) (alpha = exp(g) in (0,1)).  For bf16 workloads q, k, v
  are then rounded to bf16 on the host, so the oracle and the GPU consume the
  very same values.  Padded positions of a packed stream get g = 0, beta = 0,
  q = k = v = 0.

Decay regimes: "config" as above; "slow" g = -softplus(N(0,1) - 6) (mean
alpha ~ 0.996, keeps long-range state and the segment transition M away from
underflow); "none" g = 0.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = ["GdnInputs", "DecodeInputs", "round_bf16", "bf16_bits", "make_inputs",
           "packed_lengths", "make_packed_inputs", "workload", "make_decode_inputs",
           "WORKLOADS", "make_cotangents"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    bits = (bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))) \
        & np.uint32(0xFFFF0000)
    return bits.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e)).astype(np.float32)


def _neg_softplus(x: np.ndarray) -> np.ndarray:
    return (-np.logaddexp(np.float32(0.0), x)).astype(np.float32)


@dataclass
class GdnInputs:
    """One forward-pass workload.  Arrays are fp32 holding dtype-exact values.

    Batch layout: q,k [B,S,H,K], v [B,S,H,V], g,beta [B,S,H], h0 [B,H,K,V].
    Packed layout (cu_seqlens set, B == 1): the same arrays with B = 1 over the
    T packed tokens, h0 [N,H,K,V].
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    h0: Optional[np.ndarray]
    dtype: str
    C: int
    cu_seqlens: Optional[np.ndarray] = None
    seg_starts: Optional[List[int]] = None
    real_tokens: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.k.shape[0]

    @property
    def S(self):
        return self.k.shape[1]

    @property
    def H(self):
        return self.k.shape[2]

    @property
    def K(self):
        return self.k.shape[3]

    @property
    def V(self):
        return self.v.shape[3]


def _draw_tokens(rng, shape_qk, shape_v, dtype, decay):
    q = rng.standard_normal(shape_qk, dtype=np.float32)
    k = rng.standard_normal(shape_qk, dtype=np.float32)
    v = rng.standard_normal(shape_v, dtype=np.float32)
    b_logit = rng.standard_normal(shape_qk[:-1], dtype=np.float32)
    g_logit = rng.standard_normal(shape_qk[:-1], dtype=np.float32)
    q, k = _l2norm(q), _l2norm(k)
    beta = _sigmoid(b_logit)
    if decay == "config":
        g = _neg_softplus(g_logit)
    elif decay == "slow":
        g = _neg_softplus(g_logit - np.float32(6.0))
    elif decay == "none":
        g = np.zeros_like(g_logit)
    else:
        raise ValueError(f"unknown decay regime {decay!r}")
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return q, k, v, g, beta


def make_inputs(seed, B, S, H, K, V, C, dtype="bf16", h0_std=0.0, decay="config",
                n_segments=1, name=""):
    """Batch-mode workload: B equal-length sequences of S tokens."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _draw_tokens(rng, (B, S, H, K), (B, S, H, V), dtype, decay)
    h0 = None
    if h0_std > 0:
        h0 = (rng.standard_normal((B, H, K, V), dtype=np.float32) * np.float32(h0_std))
    seg = None
    if n_segments > 1:
        n_chunks = -(-S // C)
        per = -(-n_chunks // n_segments)
        seg = [r * per * C for r in range(n_segments) if r * per * C < S]
    return GdnInputs(q, k, v, g, beta, h0, dtype, C, seg_starts=seg, real_tokens=B * S,
                     name=name)


def packed_lengths(rng, n, total, median, sigma=1.0):
    """n lengths ~ lognormal(ln median, sigma), rescaled to sum to ``total``
    by largest-remainder rounding, each at least 1."""
    raw = rng.lognormal(mean=np.log(median), sigma=sigma, size=n)
    ideal = raw / raw.sum() * (total - n)
    base = np.floor(ideal).astype(np.int64)
    rem = (total - n) - base.sum()
    order = np.argsort(-(ideal - base), kind="stable")
    base[order[:rem]] += 1
    return (base + 1).astype(np.int64)


def make_packed_inputs(seed, n_seqs, total, H, K, V, C, dtype="bf16", h0_std=0.02,
                       decay="config", median=3000, pad_to_chunk=True, name=""):
    """Packed variable-length workload: n_seqs sequences end to end on one
    token axis, each padded to a multiple of C (g = 0, beta = 0, q = k = v = 0
    on the padded positions) when ``pad_to_chunk``."""
    rng = np.random.default_rng(seed)
    lens = packed_lengths(rng, n_seqs, total, median)
    padded = (-(-lens // C) * C) if pad_to_chunk else lens
    cu = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v, g, beta = _draw_tokens(rng, (1, T, H, K), (1, T, H, V), dtype, decay)
    for n in range(n_seqs):
        a, b = int(cu[n] + lens[n]), int(cu[n + 1])
        q[:, a:b] = 0
        k[:, a:b] = 0
        v[:, a:b] = 0
        g[:, a:b] = 0
        beta[:, a:b] = 0
    h0 = None
    if h0_std > 0:
        h0 = rng.standard_normal((n_seqs, H, K, V), dtype=np.float32) * np.float32(h0_std)
    return GdnInputs(q, k, v, g, beta, h0, dtype, C, cu_seqlens=cu, real_tokens=int(lens.sum()),
                     name=name, meta={"lengths": lens.tolist()})


def make_cotangents(seed, x, dhT_std=1.0):
    """Seeded loss gradients for a backward pass over workload ``x``:
    dl/do ~ N(0,1) in the layout of v (rounded to bf16 for bf16 workloads,
    zero on padded positions of a packed stream) and dl/dhT ~ N(0, dhT_std^2)
    [N,H,K,V] fp32 (None when dhT_std is 0)."""
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(x.v.shape, dtype=np.float32)
    if x.dtype == "bf16":
        do = round_bf16(do)
    if x.cu_seqlens is not None and "lengths" in x.meta:
        for n, ln in enumerate(x.meta["lengths"]):
            do[:, int(x.cu_seqlens[n]) + int(ln):int(x.cu_seqlens[n + 1])] = 0
    N = x.B if x.cu_seqlens is None else len(x.cu_seqlens) - 1
    dhT = None
    if dhT_std > 0:
        H = x.v.shape[2]                       # value (state) heads
        dhT = rng.standard_normal((N, H, x.K, x.V), dtype=np.float32) * np.float32(dhT_std)
    return do, dhT


@dataclass
class DecodeInputs:
    """Batched recurrent decode: ``steps`` fresh tokens per sequence.

    q,k [steps,B,H,K], v [steps,B,H,V], g,beta [steps,B,H], state0 [B,H,K,V].
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state0: np.ndarray
    dtype: str
    name: str = ""


def make_decode_inputs(seed, B, H, K, V, steps, dtype="bf16", state_std=0.02,
                       decay="config", name=""):
    rng = np.random.default_rng(seed)
    state0 = rng.standard_normal((B, H, K, V), dtype=np.float32) * np.float32(state_std)
    q, k, v, g, beta = _draw_tokens(rng, (steps, B, H, K), (steps, B, H, V), dtype, decay)
    return DecodeInputs(q, k, v, g, beta, state0, dtype, name=name)


# The five workloads.  Sizes can be shrunk (heads, tokens) for oracle-sized
# parity runs; the distributions stay those of the recipe above.
WORKLOADS = {
    0: "tiny fp32: B1 H2 S256 K=V=32 C16, zero initial state",
    1: "single sequence bf16: B1 H16 S4096 K=V=128 C64, initial state N(0,0.02^2)",
    2: "segment-composed bf16: B1 H32 S65536 in 4 segments, K=V=128 C64",
    3: "packed varlen bf16: 8 lognormal sequences (median 3000) totalling 32768, H32",
    4: "batched decode bf16: B256 H32 K=V=128, fp32 state, 128 steps",
}


def workload(i, H=None, S=None, decay="config", seed=None):
    """Workload ``i`` (0..3) with optional head / length overrides."""
    seed = i if seed is None else seed
    if i == 0:
        return make_inputs(seed, 1, S or 256, H or 2, 32, 32, 16, "f32", 0.0, decay,
                           name="tiny-f32")
    if i == 1:
        return make_inputs(seed, 1, S or 4096, H or 16, 128, 128, 64, "bf16", 0.02, decay,
                           name="seq4k-bf16")
    if i == 2:
        return make_inputs(seed, 1, S or 65536, H or 32, 128, 128, 64, "bf16", 0.02, decay,
                           n_segments=4, name="seq64k-4seg-bf16")
    if i == 3:
        return make_packed_inputs(seed, 8, S or 32768, H or 32, 128, 128, 64, "bf16", 0.02,
                                  decay, name="packed8-32k-bf16")
    raise ValueError("forward workloads are 0..3; decode is make_decode_inputs")
