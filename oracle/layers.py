"""The steps on either side of the core, in NumPy fp64 (test infrastructure).

Depthwise causal convolution.  The MaxText PR ("Add context parallelism to
the Gated Delta Net", section "Implementation") runs a depthwise causal conv1d
over the sequence before the core and exchanges exactly kernel_dim - 1 tokens
between neighbouring shards; "RFC(qwen35): TP Phase 2", section "Partition
Contract", keeps a per-request conv state of qkv_dim x (kernel_dim - 1).  The
pages give no formula; the reading taken is the plain depthwise causal
convolution, each channel c of x convolved with its own W taps,

    y[t, c] = act( sum_{i=0}^{W-1} w[c, i] x[t - (W-1) + i, c] ),

where positions before the sequence start come from the state (the W-1
previous tokens, oldest first; zeros when there is none), act is the identity
or SiLU(u) = u / (1 + exp(-u)), and the state after the sequence is its last
W-1 positions.

Gated RMSNorm.  The same RFC (section "Execution Contract") runs a gated
RMSNorm and the output gate after the core.  The reading taken: each value-head vector o of V
elements is divided by its root mean square, scaled by a weight vector, and
multiplied by SiLU of the gate z,

    y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z).
"""
import numpy as np


def silu(u):
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


def causal_conv1d(x, weight, state=None, activation="silu"):
    """One sequence: x [T, D], weight [D, W], state [D, W-1] or None.
    Returns (y [T, D], new state [D, W-1]) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    T, D = x.shape
    W = w.shape[1]
    prev = np.zeros((W - 1, D)) if state is None else np.asarray(state, dtype=np.float64).T
    ext = np.concatenate([prev, x], axis=0)          # [W-1+T, D], position t at row t + W - 1
    y = np.zeros((T, D))
    for t in range(T):
        for i in range(W):
            y[t] += w[:, i] * ext[t + i]
    if activation == "silu":
        y = silu(y)
    elif activation not in (None, "none"):
        raise ValueError(activation)
    return y, ext[T:].T.copy() if W > 1 else np.zeros((D, 0))


def causal_conv1d_packed(x, weight, cu_seqlens, state=None, activation="silu"):
    """Sequences laid end to end on x [T, D] (offsets cu_seqlens); state
    [N, D, W-1] or None.  Returns (y [T, D], states [N, D, W-1])."""
    x = np.asarray(x)
    N = len(cu_seqlens) - 1
    W = np.asarray(weight).shape[1]
    y = np.zeros(x.shape)
    st = np.zeros((N, x.shape[1], W - 1))
    for n in range(N):
        a, b = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        y[a:b], st[n] = causal_conv1d(x[a:b], weight, None if state is None else state[n], activation)
    return y, st


def gated_rmsnorm(o, weight, z=None, eps=1e-6):
    """o [..., V] normalised over its last axis, times weight [V], times
    SiLU(z) when z is given."""
    o = np.asarray(o, dtype=np.float64)
    y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * np.asarray(weight, dtype=np.float64)
    if z is not None:
        y = y * silu(z)
    return y
