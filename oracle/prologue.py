"""fp64 CPU oracle of the layer's prologue in front of the recurrence.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the benchmark's check
code; never by the library or its binding.  Plain numpy in float64, written
as the definition reads, with no blocking or fusion.

What it computes ("A Node-by-Node White-Box Walkthrough of a Quantized Hybrid
Gated DeltaNet Language Model", Principais Contribuicoes: the token's path
through a GDN sublayer runs through short convolutions before the gates and
the recurrent scan; the pages give no width and no formula, so the plainest
reading of a short causal convolution is used, with the width a parameter):

  * x [T, C] holds, per token, the channels of q (h_k*d_k), k (h_k*d_k) and
    v (h_v*d_v), in that order.
  * Depthwise causal convolution of width W per channel c, within each
    sequence of the packed batch (cu_seqlens), followed by SiLU:
        y[t, c] = SiLU(bias[c] + sum_{j=0}^{W-1} w[c, j] * xe[t - (W-1) + j, c])
    where xe is the sequence's input extended on the left by W-1 positions:
    the sequence's initial convolution state [C, W-1] (oldest first), or
    zeros.
  * q and k are then L2-normalized per (token, head) over their d_k
    channels: y / sqrt(sum y^2 + eps).  v is left as is.
  * The final convolution state of a sequence is its last W-1 extended
    inputs (oldest first), so a later call continues the convolution.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def silu(x):
    """x * sigmoid(x), in fp64."""
    return x / (1.0 + np.exp(-x))


def causal_conv(x, w, bias=None, *, cu_seqlens=None, initial_state=None,
                activation=True):
    """Depthwise causal convolution (+ SiLU) over packed sequences.

    x: [T, C]; w: [C, W]; bias: [C] or None; cu_seqlens: N+1 offsets (None =
    one sequence); initial_state: [N, C, W-1] or None (zeros).
    Returns (y [T, C], final_state [N, C, W-1])."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    T, C = x.shape
    W = w.shape[1]
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    s0 = None if initial_state is None else _f64(initial_state)
    y = np.zeros((T, C))
    final = np.zeros((N, C, W - 1))
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        head = s0[n].T if s0 is not None else np.zeros((W - 1, C))  # [W-1, C]
        xe = np.concatenate([head, x[a:b]], axis=0)  # [W-1 + L, C]
        for t in range(b - a):
            acc = np.zeros(C) if bias is None else bias.copy()
            for j in range(W):
                acc = acc + w[:, j] * xe[t + j]
            y[a + t] = silu(acc) if activation else acc
        final[n] = xe[xe.shape[0] - (W - 1):].T if W > 1 else final[n]
    return y, final


def l2norm_heads(y, d, eps):
    """Per (token, head) L2 normalization over groups of d channels."""
    y = _f64(y)
    T, C = y.shape
    h = y.reshape(T, C // d, d)
    return (h / np.sqrt(np.sum(h * h, axis=-1, keepdims=True) + eps)).reshape(T, C)


def prologue(x, w, bias, *, h_k, h_v, d_k, d_v, cu_seqlens=None,
             initial_state=None, eps=1e-6):
    """The whole prologue: returns (q [T, h_k, d_k], k [T, h_k, d_k],
    v [T, h_v, d_v], final_state [N, C, W-1])."""
    y, final = causal_conv(x, w, bias, cu_seqlens=cu_seqlens,
                           initial_state=initial_state)
    T = y.shape[0]
    cq = h_k * d_k
    q = l2norm_heads(y[:, :cq], d_k, eps).reshape(T, h_k, d_k)
    k = l2norm_heads(y[:, cq:2 * cq], d_k, eps).reshape(T, h_k, d_k)
    v = y[:, 2 * cq:].reshape(T, h_v, d_v)
    return q, k, v, final
