"""fp64 numpy reference of the chunked (WY / UT-transform) form of the gated
delta rule -- test-only.

It is the algebra the HIP prefill kernels implement, written plainly so that a
test can check it against the token-by-token oracle: the two agree to rounding
in exact arithmetic.  Per chunk of L tokens (chunks restart at each sequence
start; the last one may be short), with S0 the state entering the chunk,
ell_i = log a_i and G_i = sum_{s<=i} ell_s (chunk-local):

    E_ij = exp(G_i - G_j) for j <= i, else 0        (exp of a masked difference)
    A    = strict_lower(diag(b) (E o K K^T))
    T    = (I + A)^{-1}                              (UT transform)
    R    = diag(b) (V - diag(e^G) K S0^T)
    U    = T R                                       (pseudo-values)
    O    = diag(e^G) Q S0^T + (E o Q K^T) U
    S_L  = e^{G_L} S0 + (diag(e^{G_L - G}) U)^T K

Derivation: writing S_t = gamma_t S0 + sum_{j<=t} (gamma_t / gamma_j) u_j k_j^T
with gamma_t = e^{G_t} and substituting into one step of the rule gives
u_t = b_t (v_t - gamma_t S0 k_t - sum_{j<t} (gamma_t / gamma_j)(k_t . k_j) u_j),
i.e. (I + A) U = R.
"""
from __future__ import annotations

import numpy as np


def _softplus(x):
    return np.logaddexp(0.0, x)


def log_decay(g, A_log, dt_bias, gate_mode):
    if gate_mode == "direct":
        return np.asarray(g, dtype=np.float64)
    return -np.exp(A_log) * _softplus(g + dt_bias)


def write_strength(beta, gate_mode):
    if gate_mode == "direct":
        return np.asarray(beta, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-beta))


def chunk_step(S0, Q, K, V, ell, b):
    """One chunk.  S0 [d_v, d_k]; Q, K [L, d_k]; V [L, d_v]; ell, b [L]."""
    L = K.shape[0]
    G = np.cumsum(ell)
    diff = G[:, None] - G[None, :]
    lower = np.tril(np.ones((L, L), dtype=bool))
    E = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A = np.tril(b[:, None] * (E * (K @ K.T)), -1)
    Tm = np.linalg.inv(np.eye(L) + A)
    eG = np.exp(G)
    R = b[:, None] * (V - eG[:, None] * (K @ S0.T))
    U = Tm @ R
    O = eG[:, None] * (Q @ S0.T) + (E * (Q @ K.T)) @ U
    S_L = np.exp(G[-1]) * S0 + (np.exp(G[-1] - G)[:, None] * U).T @ K
    return O, S_L


def prefill_chunked(q, k, v, g, beta, A_log, dt_bias, *, cu_seqlens=None,
                    initial_state=None, chunk=64, gate_mode="raw"):
    """Same contract as the oracle's prefill, computed chunk by chunk."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64)
                        for x in (q, k, v, g, beta))
    T, h_k, d_k = q.shape
    _, h_v, d_v = v.shape
    group = h_v // h_k
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    n = len(cu) - 1
    o = np.zeros((T, h_v, d_v))
    fin = np.zeros((n, h_v, d_v, d_k))
    for s in range(n):
        for h in range(h_v):
            hk = h // group
            S = (np.zeros((d_v, d_k)) if initial_state is None else
                 np.asarray(initial_state[s, h], dtype=np.float64).copy())
            for c0 in range(cu[s], cu[s + 1], chunk):
                c1 = min(c0 + chunk, cu[s + 1])
                Al = None if gate_mode == "direct" else float(A_log[h])
                Dt = None if gate_mode == "direct" else float(dt_bias[h])
                ell = log_decay(g[c0:c1, h], Al, Dt, gate_mode)
                b = write_strength(beta[c0:c1, h], gate_mode)
                O, S = chunk_step(S, q[c0:c1, hk], k[c0:c1, hk], v[c0:c1, h],
                                  ell, b)
                o[c0:c1, h] = O
            fin[s, h] = S
    return o, fin
