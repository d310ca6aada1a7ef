"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent fact: a closed form, an invariant the pages state, exact
rational arithmetic, or brute force with explicit d x d transition matrices.
``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutations.py`` runs them on deliberately broken copies of it
(each copy must be rejected by at least one pin).

Facts used (pages by title and section):
  * "Why Gated DeltaNet Survives 4-Bit Quantization", Abstract (iii): each
    write overwrites the state along the current key direction -> with b = 1
    and a unit key, S_t k_t = v_t exactly (pin_overwrite); the recurrence
    forgets a state impulse -> the impulse response is bounded by the product
    of the decays (pin_contraction).
  * same Abstract (ii): softplus/exponential decay gate, sigmoid write gate ->
    gate closed forms (pin_gates).
  * "Red Lite dev15d", Pinned graph semantics steps 1-5: per-head RMSNorm with
    the shared weight, times SiLU(z), flattened -> tail closed forms
    (pin_tail).
  * the gated delta rule S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
    o_t = S_t q_t, evaluated here as explicit matrix products
    (pin_bruteforce*, pin_exact_rational) -- a different association from the
    oracle's row-wise evaluation.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(x, y, tol, what):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (what, x.shape, y.shape)
    err = float(np.max(np.abs(x - y))) if x.size else 0.0
    scale = max(float(np.max(np.abs(y))) if y.size else 0.0, 1e-300)
    assert err <= tol * max(scale, 1.0), "%s: max err %.3e (scale %.3e)" % (
        what, err, scale)


def _one_head(q, k, v, a, b, S0=None):
    """Oracle on a single head with DIRECT gates (g = log a, beta = b)."""
    o, fin = O.prefill(q[:, None], k[:, None], v[:, None],
                       np.log(a)[:, None], np.asarray(b, float)[:, None],
                       gate_mode="direct",
                       initial_state=None if S0 is None else S0[None, None])
    return o[:, 0], fin[0, 0]


def brute_force(q, k, v, a, b, S0):
    """Literal matrix form: S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
    o_t = S_t q_t, with the d_k x d_k transition matrix built explicitly."""
    d_k = k.shape[1]
    S = S0.copy()
    outs = []
    for t in range(k.shape[0]):
        P = a[t] * (np.eye(d_k) - b[t] * np.outer(k[t], k[t]))
        S = S @ P + b[t] * np.outer(v[t], k[t])
        outs.append(S @ q[t])
    return np.array(outs), S


def brute_force_product(k, v, a, b, S0):
    """Closed form of the final state as one sum of products:
    S_T = S_0 prod_t P_t + sum_t b_t v_t k_t^T prod_{s>t} P_s."""
    d_k = k.shape[1]
    T = k.shape[0]
    Ps = [a[t] * (np.eye(d_k) - b[t] * np.outer(k[t], k[t])) for t in range(T)]

    def prod(lo):
        M = np.eye(d_k)
        for s in range(lo, T):
            M = M @ Ps[s]
        return M
    S = S0 @ prod(0)
    for t in range(T):
        S = S + b[t] * np.outer(v[t], k[t]) @ prod(t + 1)
    return S


# --------------------------------------------------------------------------
# Recurrence pins
# --------------------------------------------------------------------------

def pin_overwrite():
    """b = 1 and ||k|| = 1: the write replaces the state along k, so
    S_t k_t = v_t for any decay and any previous state; with q = k the
    read-out returns v_t."""
    r = np.random.default_rng(11)
    T, d_k, d_v = 24, 8, 6
    k = _unit(r.standard_normal((T, d_k)))
    v = r.standard_normal((T, d_v))
    a = r.uniform(0.2, 1.0, T)
    S0 = r.standard_normal((d_v, d_k))
    o, fin = _one_head(k.copy(), k, v, a, np.ones(T), S0)
    _close(o, v, 1e-12, "overwrite: o_t = v_t")
    _close(fin @ k[-1], v[-1], 1e-12, "overwrite: S_T k_T = v_T")


def pin_identity():
    """a = 1, b = 0: nothing is written or forgotten."""
    r = np.random.default_rng(12)
    T, d_k, d_v = 17, 7, 5
    q = r.standard_normal((T, d_k))
    k = r.standard_normal((T, d_k))
    v = r.standard_normal((T, d_v))
    S0 = r.standard_normal((d_v, d_k))
    o, fin = _one_head(q, k, v, np.ones(T), np.zeros(T), S0)
    _close(fin, S0, 1e-15, "identity: S_T = S_0")
    _close(o, q @ S0.T, 1e-14, "identity: o_t = S_0 q_t")


def pin_pure_decay():
    """b = 0: S_t = (prod_{s<=t} a_s) S_0 and o_t = (prod a) S_0 q_t."""
    r = np.random.default_rng(13)
    T, d_k, d_v = 19, 6, 4
    q = r.standard_normal((T, d_k))
    k = r.standard_normal((T, d_k))
    v = r.standard_normal((T, d_v))
    a = r.uniform(0.5, 1.0, T)
    S0 = r.standard_normal((d_v, d_k))
    o, fin = _one_head(q, k, v, a, np.zeros(T), S0)
    _close(fin, np.prod(a) * S0, 1e-13, "pure decay: final state")
    _close(o, np.cumprod(a)[:, None] * (q @ S0.T), 1e-13, "pure decay: o_t")


def pin_linearity():
    """For fixed keys, queries and gates the map (S_0, V) -> (O, S_T) is
    linear."""
    r = np.random.default_rng(14)
    T, d_k, d_v = 21, 8, 8
    q = r.standard_normal((T, d_k))
    k = _unit(r.standard_normal((T, d_k)))
    a = r.uniform(0.7, 1.0, T)
    b = r.uniform(0.0, 1.0, T)
    X = (r.standard_normal((d_v, d_k)), r.standard_normal((T, d_v)))
    Y = (r.standard_normal((d_v, d_k)), r.standard_normal((T, d_v)))
    al, be = 0.75, -1.5
    ox, fx = _one_head(q, k, X[1], a, b, X[0])
    oy, fy = _one_head(q, k, Y[1], a, b, Y[0])
    oz, fz = _one_head(q, k, al * X[1] + be * Y[1], a, b,
                       al * X[0] + be * Y[0])
    _close(oz, al * ox + be * oy, 1e-12, "linearity: outputs")
    _close(fz, al * fx + be * fy, 1e-12, "linearity: final state")


def pin_contraction():
    """A state impulse D with no writes (V = 0) evolves as D prod(P_t); each
    P_t = a_t (I - b_t k k^T) has spectral norm a_t when 0 <= b_t <= 1 and
    ||k|| = 1, so ||S_T||_F <= (prod a_t) ||D||_F: the impulse is forgotten.
    With b = 0 the bound is attained exactly."""
    r = np.random.default_rng(15)
    T, d_k, d_v = 300, 8, 8
    k = _unit(r.standard_normal((T, d_k)))
    q = _unit(r.standard_normal((T, d_k)))
    a = r.uniform(0.9, 1.0, T)
    b = r.uniform(0.0, 1.0, T)
    D = r.standard_normal((d_v, d_k))
    _, fin = _one_head(q, k, np.zeros((T, d_v)), a, b, D)
    bound = np.prod(a) * np.linalg.norm(D)
    assert np.linalg.norm(fin) <= bound * (1 + 1e-12), (
        "contraction bound violated", np.linalg.norm(fin), bound)
    assert np.linalg.norm(fin) < 0.5 * bound, "impulse not attenuated by writes"
    _, fin0 = _one_head(q, k, np.zeros((T, d_v)), a, np.zeros(T), D)
    _close(np.linalg.norm(fin0), bound, 1e-12, "contraction: b = 0 equality")


def pin_recall():
    """Orthonormal keys, a = 1, b = 1: S = sum_j v_j e_j^T, so a query along
    e_j reads back v_j."""
    r = np.random.default_rng(16)
    d_k, d_v = 8, 5
    Qm, _ = np.linalg.qr(r.standard_normal((d_k, d_k)))
    keys = Qm.T  # rows orthonormal
    v = r.standard_normal((d_k, d_v))
    o, fin = _one_head(keys.copy(), keys, v, np.ones(d_k), np.ones(d_k))
    _close(fin, v.T @ keys, 1e-13, "recall: S = sum v_j k_j^T")
    _close(fin @ keys.T, v.T, 1e-13, "recall: S k_j = v_j")


def pin_bruteforce():
    """Explicit d x d transition matrices on small random inputs with
    non-unit keys, against both the step-by-step matrix form and the
    sum-of-products closed form."""
    r = np.random.default_rng(17)
    for (T, d_k, d_v) in [(1, 3, 2), (5, 4, 4), (12, 5, 3), (16, 8, 7)]:
        q = r.standard_normal((T, d_k))
        k = r.standard_normal((T, d_k)) * 0.6
        v = r.standard_normal((T, d_v))
        a = r.uniform(0.3, 1.0, T)
        b = r.uniform(0.0, 1.0, T)
        S0 = r.standard_normal((d_v, d_k))
        o, fin = _one_head(q, k, v, a, b, S0)
        ob, Sb = brute_force(q, k, v, a, b, S0)
        _close(o, ob, 1e-12, "brute force: outputs T=%d" % T)
        _close(fin, Sb, 1e-12, "brute force: final state T=%d" % T)
        _close(fin, brute_force_product(k, v, a, b, S0), 1e-12,
               "sum-of-products closed form T=%d" % T)


def pin_bruteforce_packed():
    """Several packed sequences (one of them empty), initial states, and value
    heads sharing key heads: each (sequence, value head) must equal brute
    force on its own slice with key head h // (h_v / h_k)."""
    r = np.random.default_rng(18)
    h_k, h_v, d_k, d_v = 2, 4, 5, 3
    lens = [6, 0, 9, 1]
    cu = np.cumsum([0] + lens)
    T = int(cu[-1])
    q = r.standard_normal((T, h_k, d_k))
    k = _unit(r.standard_normal((T, h_k, d_k)))
    v = r.standard_normal((T, h_v, d_v))
    a = r.uniform(0.4, 1.0, (T, h_v))
    b = r.uniform(0.0, 1.0, (T, h_v))
    S0 = r.standard_normal((len(lens), h_v, d_v, d_k))
    o, fin = O.prefill(q, k, v, np.log(a), b, cu_seqlens=cu, initial_state=S0,
                       gate_mode="direct")
    for n in range(len(lens)):
        t0, t1 = cu[n], cu[n + 1]
        for h in range(h_v):
            hk = h // (h_v // h_k)
            ob, Sb = brute_force(q[t0:t1, hk], k[t0:t1, hk], v[t0:t1, h],
                                 a[t0:t1, h], b[t0:t1, h], S0[n, h])
            if t1 > t0:
                _close(o[t0:t1, h], ob, 1e-12, "packed: outputs (%d,%d)" % (n, h))
            _close(fin[n, h], Sb, 1e-12, "packed: state (%d,%d)" % (n, h))


def pin_exact_rational():
    """Exact rational arithmetic on a tiny case (Fractions): the oracle must
    agree to rounding with the exact result of the matrix form."""
    F = Fraction
    k = [[F(3, 5), F(4, 5), F(0)], [F(1, 3), F(2, 3), F(2, 3)],
         [F(0), F(1), F(0)], [F(2, 7), F(3, 7), F(6, 7)],
         [F(1, 2), F(-1, 2), F(1, 4)]]
    q = [[F(1), F(0), F(0)], [F(0), F(1), F(-1)], [F(1, 2), F(1, 2), F(1, 2)],
         [F(-1), F(2), F(0)], [F(0), F(0), F(1)]]
    v = [[F(2), F(-1)], [F(1, 2), F(3)], [F(-3, 2), F(1)], [F(0), F(5, 4)],
         [F(7, 8), F(-2)]]
    a = [F(1, 2), F(3, 4), F(1), F(7, 8), F(1, 16)]
    b = [F(1), F(1, 2), F(1, 4), F(0), F(3, 4)]
    S = [[F(1, 8), F(0), F(-1, 4)], [F(1, 2), F(1, 3), F(0)]]
    S0 = [row[:] for row in S]
    outs = []
    for t in range(5):
        P = [[a[t] * ((1 if i == j else 0) - b[t] * k[t][i] * k[t][j])
              for j in range(3)] for i in range(3)]
        S = [[sum(S[r_][m] * P[m][c] for m in range(3)) + b[t] * v[t][r_] * k[t][c]
              for c in range(3)] for r_ in range(2)]
        outs.append([sum(S[r_][c] * q[t][c] for c in range(3)) for r_ in range(2)])

    def arr(x):
        return np.array([[float(e) for e in row] for row in x])
    o, fin = _one_head(arr(q), arr(k), arr(v), np.array([float(x) for x in a]),
                       np.array([float(x) for x in b]), arr(S0))
    _close(o, arr(outs), 1e-14, "exact rational: outputs")
    _close(fin, arr(S), 1e-14, "exact rational: final state")


def load_golden(name):
    """Parse a golden fixture: 'key: v1 v2 ...' lines, '#' comments."""
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = np.array([float(x) for x in rest.split()])
    return vals


def pin_golden_handworked():
    """Hand-worked two-token example (tests/golden/handworked_d2.txt)."""
    gv = load_golden("handworked_d2.txt")
    k = gv["k"].reshape(2, 2)
    q = gv["q"].reshape(2, 2)
    v = gv["v"].reshape(2, 2)
    o, fin = _one_head(q, k, v, gv["a"], gv["b"], gv["S0"].reshape(2, 2))
    _close(o, gv["o"].reshape(2, 2), 1e-15, "golden hand-worked: outputs")
    _close(fin, gv["S2"].reshape(2, 2), 1e-15, "golden hand-worked: state")


def pin_raw_equals_direct():
    """RAW gates through the recurrence equal DIRECT gates fed with the
    oracle's own (separately pinned) a and b."""
    r = np.random.default_rng(19)
    T, h, d = 23, 3, 6
    q = _unit(r.standard_normal((T, 1, d)))
    k = _unit(r.standard_normal((T, 1, d)))
    v = r.standard_normal((T, h, d))
    g = r.standard_normal((T, h))
    beta = r.standard_normal((T, h))
    A_log = r.uniform(-2, 2, h)
    dt_bias = r.uniform(-2, 0, h)
    o, fin = O.prefill(q, k, v, g, beta, A_log, dt_bias)
    a = np.zeros((T, h))
    b = np.zeros((T, h))
    for j in range(h):
        a[:, j], b[:, j] = O.gates(g[:, j], beta[:, j], A_log[j], dt_bias[j])
    o2, fin2 = O.prefill(q, k, v, np.log(a), b, gate_mode="direct")
    _close(o, o2, 1e-13, "raw vs direct gates: outputs")
    _close(fin, fin2, 1e-13, "raw vs direct gates: state")


def pin_decode():
    """One decode step per sequence equals the explicit one-step matrix form
    S_1 = a S_0 (I - b k k^T) + b v k^T, o = S_1 q, including shared key heads."""
    r = np.random.default_rng(20)
    N, h_k, h_v, d = 3, 2, 4, 6
    q = _unit(r.standard_normal((N, h_k, d)))
    k = _unit(r.standard_normal((N, h_k, d)))
    v = r.standard_normal((N, h_v, d))
    a = r.uniform(0.1, 1.0, (N, h_v))
    b = r.uniform(0.0, 1.0, (N, h_v))
    S0 = r.standard_normal((N, h_v, d, d))
    o, S1 = O.decode(q, k, v, np.log(a), b, None, None, S0, gate_mode="direct")
    for n in range(N):
        for h in range(h_v):
            hk = h // (h_v // h_k)
            ob, Sb = brute_force(q[n, hk][None], k[n, hk][None], v[n, h][None],
                                 a[n, h][None], b[n, h][None], S0[n, h])
            _close(o[n, h], ob[0], 1e-13, "decode: output")
            _close(S1[n, h], Sb, 1e-13, "decode: state")


# --------------------------------------------------------------------------
# Gate pins (closed forms and library routines)
# --------------------------------------------------------------------------

def pin_gates():
    g0 = np.zeros(1)
    # A_log = 0, g + dt_bias = 0: a = exp(-1 * ln 2) = 1/2; beta = 0: b = 1/2.
    a, b = O.gates(g0, g0, 0.0, 0.0)
    _close(a, [0.5], 1e-15, "gate: a(0,0,0) = 1/2")
    _close(b, [0.5], 1e-15, "gate: b(0) = 1/2")
    # A_log = ln 2 doubles the rate: a = 1/4.
    a, _ = O.gates(g0, g0, math.log(2.0), 0.0)
    _close(a, [0.25], 1e-15, "gate: a with exp(A_log) = 2")
    # g + dt_bias = ln(e - 1): softplus = 1 exactly, so a = exp(-exp(A_log)).
    s = math.log(math.e - 1.0)
    a, _ = O.gates(np.array([0.3]), g0, math.log(3.0), s - 0.3)
    _close(a, [math.exp(-3.0)], 1e-14, "gate: softplus(ln(e-1)) = 1")
    # A_log -> -inf: no decay; large positive pre-activation: softplus ~ x.
    a, _ = O.gates(np.array([5.0]), g0, -60.0, 0.0)
    _close(a, [1.0], 1e-15, "gate: A_log -> -inf gives a = 1")
    a, _ = O.gates(np.array([40.0]), g0, math.log(0.01), 0.0)
    _close(a, [math.exp(-0.4)], 1e-14, "gate: softplus(40) = 40")
    # Large negative pre-activation: softplus(x) ~ e^x, so a ~ exp(-e^x).
    a, _ = O.gates(np.array([-30.0]), g0, 0.0, 0.0)
    _close(a, [math.exp(-math.exp(-30.0))], 1e-15, "gate: softplus(-30)")
    # beta -> +-inf saturates the sigmoid.
    _, b = O.gates(np.zeros(2), np.array([60.0, -60.0]), 0.0, 0.0)
    _close(b, [1.0, math.exp(-60.0)], 1e-15, "gate: sigmoid saturation")
    # Against library routines on random inputs.
    from scipy.special import expit
    r = np.random.default_rng(21)
    g = r.standard_normal(200) * 3
    beta = r.standard_normal(200) * 4
    for A_log, dt in [(0.7, -1.3), (-2.0, 0.0), (2.5, -0.2)]:
        a, b = O.gates(g, beta, A_log, dt)
        _close(np.log(a), -math.exp(A_log) * np.logaddexp(0.0, g + dt), 1e-13,
               "gate: log a vs numpy logaddexp")
        _close(b, expit(beta), 1e-15, "gate: b vs scipy expit")
    # DIRECT mode passes the values through.
    a, b = O.gates(np.array([math.log(0.3)]), np.array([0.8]), gate_mode="direct")
    _close(a, [0.3], 1e-15, "gate: direct a")
    _close(b, [0.8], 1e-15, "gate: direct b")


# --------------------------------------------------------------------------
# Tail pins (closed forms)
# --------------------------------------------------------------------------

def _silu(z):
    from scipy.special import expit
    return z * expit(z)


def pin_tail():
    d = 128
    eps = 1e-6
    ones = np.ones(d)
    # A constant head o = c * 1 with unit weight normalises to
    # sign(c) / sqrt(1 + eps / c^2); z enters only through SiLU(z).
    r = np.random.default_rng(22)
    z = r.standard_normal(d)
    for c in [2.0, -0.5, 1e-3, -3e-3]:
        y = O.gated_rmsnorm(c * ones[None], z[None], ones, eps)[0]
        want = math.copysign(1.0, c) / math.sqrt(1.0 + eps / (c * c)) * _silu(z)
        _close(y, want, 1e-14, "tail: constant head c=%g" % c)
    # z = 0 kills the output; SiLU(1) = 1 / (1 + e^-1).
    x = r.standard_normal((3, d))
    _close(O.gated_rmsnorm(x, np.zeros((3, d)), ones, eps), np.zeros((3, d)),
           0.0, "tail: z = 0")
    y = O.gated_rmsnorm(np.full((1, d), 5.0), np.ones((1, d)), ones, 0.0)
    _close(y, np.full((1, d), 1.0 / (1.0 + math.exp(-1.0))), 1e-15,
           "tail: SiLU(1)")
    # eps = 0: the normalised head has unit mean square; scale invariance,
    # odd symmetry and linearity in the weight.
    w = r.uniform(0.5, 1.5, d)
    zz = r.standard_normal((3, d))
    y = O.gated_rmsnorm(x, zz, ones, 0.0) / _silu(zz)
    _close(np.mean(y * y, axis=1), np.ones(3), 1e-14, "tail: unit mean square")
    _close(O.gated_rmsnorm(7.5 * x, zz, w, 0.0), O.gated_rmsnorm(x, zz, w, 0.0),
           1e-14, "tail: scale invariance")
    _close(O.gated_rmsnorm(-x, zz, w, eps), -O.gated_rmsnorm(x, zz, w, eps),
           1e-15, "tail: odd in o")
    _close(O.gated_rmsnorm(x, zz, 2.0 * w, eps),
           2.0 * O.gated_rmsnorm(x, zz, w, eps), 1e-15, "tail: linear in w")
    # Head-major flatten: head h of token t lands at [t, h*d : (h+1)*d].
    o = r.standard_normal((2, 4, d))
    zt = r.standard_normal((2, 4, d))
    flat = O.tail(o, zt, w, eps)
    assert flat.shape == (2, 4 * d)
    for t in range(2):
        for h in range(4):
            _close(flat[t, h * d:(h + 1) * d],
                   O.gated_rmsnorm(o[t, h][None], zt[t, h][None], w, eps)[0],
                   0.0, "tail: flatten head-major")


ALL_PINS = [pin_overwrite, pin_identity, pin_pure_decay, pin_linearity,
            pin_contraction, pin_recall, pin_bruteforce, pin_bruteforce_packed,
            pin_exact_rational, pin_golden_handworked, pin_raw_equals_direct,
            pin_decode, pin_gates, pin_tail]
