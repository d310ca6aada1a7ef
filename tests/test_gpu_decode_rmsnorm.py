"""GPU parity of gdn_decode_step and gdn_gated_rmsnorm against the fp64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from parity import (TOL_BF16_INPUTS, TOL_F32_INPUTS, bf16_ulp_diff,
                    per_state_rel, rel_inf, rowwise_rel)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode_case(N, h_k, h_v, d_k, io, seed, tail=True, s0_std=0.05,
                 gates="spread"):
    wl = I.Workload("dec", [1] * N, h_k, h_v, d_k, d_k, io=io, gates=gates,
                    tail=tail, s0_std=s0_std, seed=seed, decode=True)
    return I.make_inputs(wl, device=DEV)


def _oracle_decode(x, tail):
    o, st = O.decode(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias, x.s0)
    if tail:
        o = O.tail(o, x.z, x.w, x.eps)
    return o, st


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("tail", [False, True])
def test_decode_small(d, io, tail):
    x = _decode_case(5, 2, 4, d, io, seed=100 + d, tail=tail)
    st = x.s0.clone()
    out = G.gdn_decode_step(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                            st, z=x.z if tail else None, norm_weight=x.w,
                            eps=x.eps, out_dtype=torch.float32)
    o_ref, st_ref = _oracle_decode(x, tail)
    tol = TOL_F32_INPUTS if io == "f32" else TOL_BF16_INPUTS
    e_o = rel_inf(out.reshape(o_ref.shape), o_ref)
    e_s = per_state_rel(st, st_ref)
    print("decode d=%d io=%s tail=%d: out %.2e state %.2e" % (d, io, tail,
                                                             e_o, e_s))
    assert e_o <= tol and e_s <= tol


def test_decode_direct_gates_and_bf16_out():
    x = _decode_case(7, 2, 2, 64, "bf16", seed=7, tail=True)
    a = torch.rand(7, 2, device=DEV) * 0.9 + 0.05
    b = torch.rand(7, 2, device=DEV)
    g = torch.log(a)
    st1, st2 = x.s0.clone(), x.s0.clone()
    o32 = G.gdn_decode_step(x.q, x.k, x.v, g, b, None, None, st1, z=x.z,
                            norm_weight=x.w, gate_mode="direct",
                            out_dtype=torch.float32)
    o16 = G.gdn_decode_step(x.q, x.k, x.v, g, b, None, None, st2, z=x.z,
                            norm_weight=x.w, gate_mode="direct")
    assert o16.dtype == torch.bfloat16
    assert bf16_ulp_diff(o16, o32) <= 1
    assert torch.equal(st1, st2)
    o_ref, st_ref = O.decode(x.q, x.k, x.v, g, b, None, None, x.s0,
                             gate_mode="direct")
    o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    assert rel_inf(o32.reshape(o_ref.shape), o_ref) <= TOL_BF16_INPUTS
    assert per_state_rel(st1, st_ref) <= TOL_BF16_INPUTS


def test_decode_batched_full_size():
    """256 sequences x 32 value heads (16 key heads), d = 128, fp32 state
    [256, 32, 128, 128] updated in place, fused tail; every head checked."""
    wl = I.WORKLOADS["decode_n256_hv32"]
    x = I.make_inputs(wl, device=DEV)
    st = x.s0.clone()
    out = G.gdn_decode_step(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                            st, z=x.z, norm_weight=x.w, eps=x.eps,
                            out_dtype=torch.float32)
    o_ref, st_ref = _oracle_decode(x, True)
    e_o = rowwise_rel(out, o_ref, 128)          # every (sequence, head)
    e_s = rowwise_rel(st, st_ref, 128 * 128)    # every head's state
    print("decode full: out %.2e state %.2e" % (e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS
    # bf16 output of a second identical step equals RNE of the fp32 output.
    st2 = x.s0.clone()
    out16 = G.gdn_decode_step(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                              st2, z=x.z, norm_weight=x.w, eps=x.eps)
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(st2, st)


def test_decode_repeated_equals_prefill_oracle():
    """Several decode steps carried through the state equal one oracle prefill
    of the same tokens."""
    T, h_k, h_v, d = 9, 2, 4, 32
    x = I.random_case(T_list=[T], h_k=h_k, h_v=h_v, d_k=d, d_v=d, io="f32",
                      seed=3, s0_std=0.1, device=DEV)
    st = x.s0.clone()  # [1, h_v, d, d]
    outs = []
    for t in range(T):
        outs.append(G.gdn_decode_step(
            x.q[t:t + 1].contiguous(), x.k[t:t + 1].contiguous(),
            x.v[t:t + 1].contiguous(), x.g[t:t + 1].contiguous(),
            x.beta[t:t + 1].contiguous(), x.A_log, x.dt_bias, st,
            out_dtype=torch.float32))
    o = torch.cat(outs)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                             initial_state=x.s0)
    assert rel_inf(o, o_ref) <= TOL_F32_INPUTS
    assert per_state_rel(st, f_ref) <= TOL_F32_INPUTS


def test_decode_empty_batch():
    x = _decode_case(1, 1, 1, 16, "f32", seed=0)
    out = G.gdn_decode_step(x.q[:0], x.k[:0], x.v[:0], x.g[:0], x.beta[:0],
                            x.A_log, x.dt_bias, x.s0[:0])
    assert out.numel() == 0


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("xdt,zdt", [(torch.float32, torch.float32),
                                     (torch.bfloat16, torch.bfloat16),
                                     (torch.float32, torch.bfloat16)])
def test_rmsnorm(d, xdt, zdt):
    gen = torch.Generator(device=DEV).manual_seed(d)
    rows = 1037
    x = torch.randn(rows, d, generator=gen, device=DEV).to(xdt)
    z = torch.randn(rows, d, generator=gen, device=DEV).to(zdt)
    w = torch.rand(d, generator=gen, device=DEV) + 0.5
    y = G.gdn_gated_rmsnorm(x, z, w, 1e-6, out_dtype=torch.float32)
    ref = O.gated_rmsnorm(x, z, w, 1e-6)
    assert rel_inf(y, ref) <= 1e-5
    y16 = G.gdn_gated_rmsnorm(x, z, w, 1e-6, out_dtype=torch.bfloat16)
    assert bf16_ulp_diff(y16, y) <= 1


def test_rmsnorm_in_place_and_empty():
    gen = torch.Generator(device=DEV).manual_seed(1)
    x = torch.randn(300, 128, generator=gen, device=DEV)
    z = torch.randn(300, 128, generator=gen, device=DEV)
    w = torch.rand(128, generator=gen, device=DEV) + 0.5
    ref = O.gated_rmsnorm(x, z, w, 1e-6)
    G.gdn_gated_rmsnorm(x, z, w, 1e-6, out=x)
    assert rel_inf(x, ref) <= 1e-5
    e = torch.empty(0, 128, device=DEV)
    assert G.gdn_gated_rmsnorm(e, e.clone(), w).numel() == 0
