"""The chunked WY/UT form that the HIP prefill kernels implement equals the
token-by-token oracle (fp64, both on the CPU), for chunk sizes 1, 16 and 64,
lengths that are not multiples of the chunk, packed sequences, carried state,
shared key heads and strong decay."""
import numpy as np
import pytest

import chunked_ref as CR
from oracle import oracle as O


def _case(seed, lens, h_k, h_v, d, A_range, s0=True):
    r = np.random.default_rng(seed)
    T = sum(lens)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(r.standard_normal((T, h_k, d)))
    k = unit(r.standard_normal((T, h_k, d)))
    v = r.standard_normal((T, h_v, d))
    g = r.standard_normal((T, h_v))
    beta = r.standard_normal((T, h_v))
    A_log = r.uniform(*A_range, h_v)
    dt_bias = r.uniform(-2, 0, h_v)
    S0 = r.standard_normal((len(lens), h_v, d, d)) * 0.05 if s0 else None
    cu = np.cumsum([0] + list(lens))
    return q, k, v, g, beta, A_log, dt_bias, S0, cu


@pytest.mark.parametrize("chunk", [1, 16, 64])
@pytest.mark.parametrize("lens,h_k,h_v,d,A_range", [
    ([67], 1, 1, 16, (0.0, np.log(16.0))),     # strong decay (log a to -49)
    ([130, 0, 5, 64], 2, 4, 8, (-7.0, 2.3)),   # packed, shared key heads
    ([200], 1, 2, 32, (-7.0, 0.0)),            # mild decay, longer chain
])
def test_chunked_equals_sequential(chunk, lens, h_k, h_v, d, A_range):
    q, k, v, g, beta, A_log, dt_bias, S0, cu = _case(
        7 + chunk, lens, h_k, h_v, d, A_range)
    o_ref, f_ref = O.prefill(q, k, v, g, beta, A_log, dt_bias, cu_seqlens=cu,
                             initial_state=S0)
    o_ch, f_ch = CR.prefill_chunked(q, k, v, g, beta, A_log, dt_bias,
                                    cu_seqlens=cu, initial_state=S0,
                                    chunk=chunk)
    scale_o = max(np.abs(o_ref).max(), 1.0)
    scale_s = max(np.abs(f_ref).max(), 1.0)
    assert np.abs(o_ch - o_ref).max() <= 1e-11 * scale_o
    assert np.abs(f_ch - f_ref).max() <= 1e-11 * scale_s
