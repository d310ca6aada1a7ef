"""Pins of the prologue oracle (oracle/prologue.py) against facts that do not
come from the oracle itself: numpy's own convolution, the causal and
per-sequence structure of the definition, continuation through the carried
state, the algebra of SiLU, and the unit norm of normalized heads."""
import numpy as np
import pytest

from oracle import prologue as P

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_conv_equals_numpy_convolve():
    """Zero initial state, one sequence: each channel is np.convolve of the
    input with the reversed taps, truncated to the causal part."""
    T, C, W = 23, 5, 4
    x, w, b = _rand(T, C), _rand(C, W), _rand(C)
    y, _ = P.causal_conv(x, w, b, activation=False)
    for c in range(C):
        ref = np.convolve(x[:, c], w[c, ::-1])[:T] + b[c]
        assert np.allclose(y[:, c], ref, rtol=0, atol=1e-12)


def test_width_one_is_pointwise_silu():
    x = _rand(9, 3)
    w = np.ones((3, 1))
    y, fin = P.causal_conv(x, w)
    assert np.allclose(y, x * (1.0 / (1.0 + np.exp(-x))), atol=1e-15)
    assert fin.shape == (1, 3, 0)


def test_silu_identities():
    x = np.linspace(-30, 30, 61)
    s = P.silu(x)
    assert s[30] == 0.0                                  # SiLU(0) = 0
    assert np.allclose(P.silu(-x), s - x, atol=1e-12)    # SiLU(-x) = SiLU(x) - x
    assert abs(P.silu(np.array([40.0]))[0] - 40.0) < 1e-12


def test_causal_and_local():
    """Changing x at token t changes only tokens t .. t+W-1 of the same
    sequence."""
    T, C, W = 20, 4, 3
    x, w = _rand(T, C), _rand(C, W)
    y0, _ = P.causal_conv(x, w)
    x2 = x.copy()
    x2[7] += 1.0
    y1, _ = P.causal_conv(x2, w)
    changed = np.where(np.abs(y1 - y0).max(axis=1) > 0)[0]
    assert changed.min() == 7 and changed.max() <= 7 + W - 1


def test_packed_equals_separate_and_state_continues():
    """Packing sequences equals running them one by one, and splitting one
    sequence in two pieces, carrying the final state, equals one run."""
    C, W = 6, 4
    lens = [5, 0, 2, 11]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x, w, b = _rand(cu[-1], C), _rand(C, W), _rand(C)
    s0 = _rand(len(lens), C, W - 1)
    y, fin = P.causal_conv(x, w, b, cu_seqlens=cu, initial_state=s0)
    for n in range(len(lens)):
        yn, fn = P.causal_conv(x[cu[n]:cu[n + 1]], w, b,
                               initial_state=s0[n:n + 1])
        assert np.array_equal(yn, y[cu[n]:cu[n + 1]])
        assert np.array_equal(fn[0], fin[n])
    # the empty sequence hands its initial state through
    assert np.array_equal(fin[1], s0[1])
    # split the 11-token sequence after 4 tokens
    a = cu[3]
    y1, f1 = P.causal_conv(x[a:a + 4], w, b, initial_state=s0[3:4])
    y2, f2 = P.causal_conv(x[a + 4:a + 11], w, b, initial_state=f1)
    assert np.allclose(np.concatenate([y1, y2]), y[a:a + 11], atol=1e-14)
    assert np.allclose(f2[0], fin[3], atol=0)


def test_final_state_is_last_inputs():
    T, C, W = 8, 3, 4
    x = _rand(T, C)
    _, fin = P.causal_conv(x, _rand(C, W))
    assert np.array_equal(fin[0], x[T - (W - 1):].T)


def test_prologue_heads_unit_norm_and_split():
    T, h_k, h_v, d = 7, 2, 4, 16
    C = 2 * h_k * d + h_v * d
    x, w, b = _rand(T, C) * 3, _rand(C, 4), _rand(C)
    q, k, v, _ = P.prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d, eps=0.0)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-12)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-12)
    y, _ = P.causal_conv(x, w, b)
    assert np.array_equal(v.reshape(T, -1), y[:, 2 * h_k * d:])
    # q is y's first h_k*d channels scaled per head (direction kept)
    yq = y[:, :h_k * d].reshape(T, h_k, d)
    cos = np.sum(yq * q, -1) / np.linalg.norm(yq, axis=-1)
    assert np.allclose(cos, 1.0, atol=1e-12)


@pytest.mark.parametrize("eps", [1e-6, 1.0])
def test_l2norm_eps_inside_root(eps):
    y = np.full((1, 4), 0.5)            # sum of squares = 1
    out = P.l2norm_heads(y, 4, eps)
    assert np.allclose(out, 0.5 / np.sqrt(1.0 + eps), atol=1e-15)
