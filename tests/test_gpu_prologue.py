"""GPU parity of gdn_conv_prologue (causal convolution + SiLU over the q, k,
v channels, per-head L2 normalization of q and k, carried convolution
state) against the fp64 prologue oracle, through the C ABI; and the
prologue feeding the chunked prefill end to end."""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from oracle import prologue as P
from parity import (TOL_BF16_INPUTS, TOL_F32_INPUTS, bf16_ulp_diff,
                    per_head_rel, rel_inf, rowwise_rel)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(lens, h_k, h_v, d, W, io, seed, bias=True, state=True):
    """x ~ N(0, 1), taps ~ N(0, 1/W), bias ~ N(0, 0.1), states ~ N(0, 1)."""
    gen = torch.Generator(device=DEV).manual_seed(seed)
    C = 2 * h_k * d + h_v * d
    T = int(sum(lens))
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    x = torch.randn(T, C, generator=gen, device=DEV).to(dt)
    w = torch.randn(C, W, generator=gen, device=DEV) / np.sqrt(W)
    b = 0.1 * torch.randn(C, generator=gen, device=DEV) if bias else None
    N = len(lens)
    s0 = (torch.randn(N, C, W - 1, generator=gen, device=DEV)
          if state else None)
    cu_list = [0] + list(np.cumsum(lens))
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    return x, w, b, s0, cu, cu_list


def _check(x, w, b, s0, cu, cu_list, h_k, h_v, d, tol, out_dtype=torch.float32):
    q, k, v, fin = G.gdn_conv_prologue(
        x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d, cu_seqlens=cu,
        cu_seqlens_host=cu_list, initial_conv_state=s0,
        output_final_state=True, eps=1e-6, out_dtype=out_dtype)
    qr, kr, vr, fr = P.prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d,
                                cu_seqlens=cu_list, initial_state=s0, eps=1e-6)
    if x.shape[0]:
        e = max(rowwise_rel(q, qr, d), rowwise_rel(k, kr, d),
                rowwise_rel(v, vr, d))
    else:
        e = 0.0
    e_s = rel_inf(fin, fr) if fin.numel() else 0.0
    return e, e_s, (q, k, v, fin)


@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prologue_small(W, d, io):
    lens = [37, 0, 3, 70, 1]           # ragged, empty, shorter than W, > 2 tiles
    h_k, h_v = 2, 4
    x, w, b, s0, cu, cu_list = _inputs(lens, h_k, h_v, d, W, io,
                                       seed=W * 100 + d)
    tol = TOL_F32_INPUTS if io == "f32" else TOL_BF16_INPUTS
    e, e_s, _ = _check(x, w, b, s0, cu, cu_list, h_k, h_v, d, tol)
    print("prologue W=%d d=%d io=%s: out %.2e state %.2e" % (W, d, io, e, e_s))
    assert e <= tol and e_s == 0.0   # the state is a copy of inputs


def test_prologue_no_bias_no_state_single_sequence():
    x, w, _, _, _, _ = _inputs([150], 1, 2, 32, 4, "bf16", seed=3)
    q, k, v, fin = G.gdn_conv_prologue(x, w, None, h_k=1, h_v=2, d_k=32,
                                       d_v=32, output_final_state=True,
                                       out_dtype=torch.float32)
    qr, kr, vr, fr = P.prologue(x, w, None, h_k=1, h_v=2, d_k=32, d_v=32)
    e = max(rowwise_rel(q, qr, 32), rowwise_rel(k, kr, 32), rowwise_rel(v, vr, 32))
    assert e <= TOL_BF16_INPUTS and rel_inf(fin, fr) == 0.0


def test_prologue_full_size_sampled():
    """The 32768-token layer's shape (16 key / 32 value heads, d = 128,
    C = 8192), width 4, bf16 in and out: the first 1024 tokens and a window
    in the middle (its state rebuilt from the inputs before it) against the
    oracle; bf16 output == RNE of the fp32 output."""
    T, h_k, h_v, d, W = 32768, 16, 32, 128, 4
    x, w, b, _, _, _ = _inputs([T], h_k, h_v, d, W, "bf16", seed=21,
                               state=False)
    q, k, v, _ = G.gdn_conv_prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d,
                                     out_dtype=torch.float32)
    q16, k16, v16, _ = G.gdn_conv_prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d,
                                           d_v=d)
    for out16, out32 in ((q16, q), (k16, k), (v16, v)):
        assert bf16_ulp_diff(out16, out32) <= 1
    for a, n in ((0, 1024), (20000, 512)):
        s0 = None
        if a:
            s0 = x[a - (W - 1):a].float().T.unsqueeze(0).contiguous()
        qr, kr, vr, _ = P.prologue(x[a:a + n], w, b, h_k=h_k, h_v=h_v, d_k=d,
                                   d_v=d, initial_state=s0)
        e = max(rowwise_rel(q[a:a + n], qr, d), rowwise_rel(k[a:a + n], kr, d),
                rowwise_rel(v[a:a + n], vr, d))
        print("prologue full tokens %d..%d: %.2e" % (a, a + n, e))
        assert e <= TOL_BF16_INPUTS


def test_prologue_decode_continuation():
    """A prefill-sized call followed by one-token-per-sequence calls that
    carry the convolution state equals one call over all the tokens."""
    lens, extra = [9, 2, 40], 3
    h_k, h_v, d, W = 1, 2, 64, 4
    tot = [L + extra for L in lens]
    x, w, b, s0, _, _ = _inputs(tot, h_k, h_v, d, W, "f32", seed=8)
    cu_t = [0] + list(np.cumsum(tot))
    full = G.gdn_conv_prologue(
        x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d,
        cu_seqlens=torch.tensor(cu_t, dtype=torch.int32, device=DEV),
        initial_conv_state=s0, output_final_state=True)
    head = torch.cat([x[cu_t[n]:cu_t[n] + lens[n]] for n in range(3)])
    cu_h = [0] + list(np.cumsum(lens))
    _, _, _, st = G.gdn_conv_prologue(
        head.contiguous(), w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d,
        cu_seqlens=torch.tensor(cu_h, dtype=torch.int32, device=DEV),
        initial_conv_state=s0, output_final_state=True)
    one = torch.arange(4, dtype=torch.int32, device=DEV)
    for j in range(extra):
        xt = torch.stack([x[cu_t[n] + lens[n] + j] for n in range(3)]).contiguous()
        qd, kd, vd, st2 = G.gdn_conv_prologue(
            xt, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d, cu_seqlens=one,
            initial_conv_state=st, output_final_state=True)
        for n in range(3):
            t = cu_t[n] + lens[n] + j
            assert torch.equal(qd[n], full[0][t]) and torch.equal(vd[n], full[2][t])
        st = st2
    assert torch.equal(st, full[3])


def test_prologue_feeds_prefill():
    """The path from the projected channels to the recurrent output: the
    prologue's bf16 q, k, v fed to the bf16 matrix-core prefill, against the
    oracle prologue followed by the oracle recurrence."""
    T, h_k, h_v, d = 300, 2, 4, 128
    x, w, b, _, _, _ = _inputs([T], h_k, h_v, d, 4, "bf16", seed=13,
                               state=False)
    gen = torch.Generator(device=DEV).manual_seed(14)
    g = torch.randn(T, h_v, generator=gen, device=DEV)
    beta = torch.randn(T, h_v, generator=gen, device=DEV)
    A_log = torch.log(torch.linspace(1.0, 8.0, h_v, device=DEV))
    dt_bias = -torch.rand(h_v, generator=gen, device=DEV)
    q, k, v, _ = G.gdn_conv_prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d)
    out, fin = G.gdn_chunk_prefill(q, k, v, g, beta, A_log, dt_bias,
                                   chunk_size=64, out_dtype=torch.float32)
    # The prologue itself: fp32 outputs against the oracle, and the bf16
    # outputs the prefill consumed within one ulp of their rounding.
    q32, k32, v32, _ = G.gdn_conv_prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d,
                                           d_v=d, out_dtype=torch.float32)
    qr, kr, vr, _ = P.prologue(x, w, b, h_k=h_k, h_v=h_v, d_k=d, d_v=d)
    e_p = max(rowwise_rel(q32, qr, d), rowwise_rel(k32, kr, d),
              rowwise_rel(v32, vr, d))
    assert e_p <= TOL_BF16_INPUTS
    for a16, a32 in ((q, q32), (k, k32), (v, v32)):
        assert bf16_ulp_diff(a16, a32) <= 1
    # The recurrence on exactly the values the kernel consumed.
    o_ref, f_ref = O.prefill(q, k, v, g, beta, A_log, dt_bias)
    e_o = per_head_rel(out, o_ref, [0, T], h_v, d)
    e_s = rel_inf(fin[0], f_ref[0])
    print("prologue -> prefill: prologue %.2e out %.2e state %.2e" % (e_p, e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS
