"""GPU parity of gdn_chunk_prefill against the fp64 token-by-token oracle,
through the C ABI: small shapes spanning several chunks with ragged tails,
packed sequences (including empty ones), carried state, shared key heads,
the fused tail, and the bf16 / fp32 output contract."""
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from parity import (TOL_BF16_INPUTS, TOL_F32_INPUTS, bf16_ulp_diff,
                    per_head_rel, per_state_rel)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_gpu(x, chunk, tail, out_dtype=torch.float32, s0=True, **kw):
    return G.gdn_chunk_prefill(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
        cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_list,
        initial_state=x.s0 if s0 else None, z=x.z if tail else None,
        norm_weight=x.w, eps=x.eps, chunk_size=chunk, out_dtype=out_dtype,
        **kw)


def run_oracle(x, tail, s0=True):
    o, f = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                     cu_seqlens=x.cu_list,
                     initial_state=x.s0 if s0 else None)
    if tail:
        o = O.tail(o, x.z, x.w, x.eps)
    return o, f


def check(x, chunk, tail, tol, s0=True, label=""):
    out, fin = run_gpu(x, chunk, tail, s0=s0)
    o_ref, f_ref = run_oracle(x, tail, s0=s0)
    h_v, d_v = x.v.shape[1], x.v.shape[2]
    e_o = per_head_rel(out, o_ref, x.cu_list, h_v, d_v)
    e_s = per_state_rel(fin, f_ref)
    print("%s chunk=%d tail=%d: out %.2e state %.2e" % (label, chunk, tail,
                                                       e_o, e_s))
    assert e_o <= tol, (label, e_o)
    assert e_s <= tol, (label, e_s)
    return out, fin


def test_tiny_fp32_workload():
    """B=1, T=64, H=2, d=16, fp32, chunk 16, strong decay gates."""
    wl = I.WORKLOADS["tiny_fp32"]
    x = I.make_inputs(wl, device=DEV)
    check(x, wl.chunk, False, TOL_F32_INPUTS, s0=False, label="tiny")


CASES = [
    # lens, h_k, h_v, d, chunk, io, tail, gates
    ([1], 1, 1, 16, 16, "f32", False, "tiny"),
    ([15], 1, 2, 16, 16, "f32", True, "tiny"),
    ([17, 16, 0, 63], 2, 2, 32, 16, "f32", False, "spread"),
    ([64, 65], 1, 2, 64, 32, "f32", True, "spread"),
    ([200], 2, 4, 64, 64, "f32", False, "tiny"),
    ([130, 7], 1, 1, 128, 64, "f32", True, "spread"),
    ([100, 0, 29], 2, 4, 32, 32, "bf16", True, "spread"),
    ([77], 1, 2, 64, 16, "bf16", False, "tiny"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_generic_shapes(case):
    lens, h_k, h_v, d, chunk, io, tail, gates = case
    x = I.random_case(T_list=lens, h_k=h_k, h_v=h_v, d_k=d, d_v=d, io=io,
                      seed=sum(lens) + d, gates=gates, tail=tail,
                      s0_std=0.05, device=DEV)
    tol = TOL_F32_INPUTS if io == "f32" else TOL_BF16_INPUTS
    check(x, chunk, tail, tol, label=str(case))


def test_bf16_out_is_rne_of_f32_out():
    x = I.random_case(T_list=[70, 33], h_k=2, h_v=4, d_k=64, d_v=64, io="bf16",
                      seed=5, tail=True, s0_std=0.05, device=DEV)
    o32, f32 = run_gpu(x, 32, True, out_dtype=torch.float32)
    o16, f16 = run_gpu(x, 32, True, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert bf16_ulp_diff(o16, o32) <= 1
    assert torch.equal(f32, f16)


def test_split_prefill_carries_state():
    """Prefill of tokens [0, 50) then [50, 120) from the carried final state
    equals one prefill of [0, 120)."""
    x = I.random_case(T_list=[120], h_k=1, h_v=2, d_k=32, d_v=32, io="f32",
                      seed=9, s0_std=0.05, device=DEV)
    o_all, f_all = run_gpu(x, 16, False)
    sl = lambda t, a, b: t[a:b].contiguous()
    o1, f1 = G.gdn_chunk_prefill(sl(x.q, 0, 50), sl(x.k, 0, 50),
                                 sl(x.v, 0, 50), sl(x.g, 0, 50),
                                 sl(x.beta, 0, 50), x.A_log, x.dt_bias,
                                 initial_state=x.s0, chunk_size=16,
                                 out_dtype=torch.float32)
    o2, f2 = G.gdn_chunk_prefill(sl(x.q, 50, 120), sl(x.k, 50, 120),
                                 sl(x.v, 50, 120), sl(x.g, 50, 120),
                                 sl(x.beta, 50, 120), x.A_log, x.dt_bias,
                                 initial_state=f1, chunk_size=16,
                                 out_dtype=torch.float32)
    o_ref, f_ref = run_oracle(x, False)
    assert per_state_rel(f2, f_ref) <= TOL_F32_INPUTS
    assert per_head_rel(torch.cat([o1, o2]), o_ref, [0, 120], 2, 32) <= TOL_F32_INPUTS
    assert per_state_rel(f_all, f_ref) <= TOL_F32_INPUTS


def test_packed_equals_separate_and_deterministic():
    lens = [40, 0, 97, 16]
    x = I.random_case(T_list=lens, h_k=2, h_v=4, d_k=64, d_v=64, io="bf16",
                      seed=11, tail=True, s0_std=0.05, device=DEV)
    out, fin = run_gpu(x, 32, True)
    out2, fin2 = run_gpu(x, 32, True)
    assert torch.equal(out, out2) and torch.equal(fin, fin2)  # bitwise
    cu = x.cu_list
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = lambda t: t[a:b].contiguous()
        o_n, f_n = G.gdn_chunk_prefill(
            sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.A_log,
            x.dt_bias, initial_state=x.s0[n:n + 1].contiguous(), z=sl(x.z),
            norm_weight=x.w, eps=x.eps, chunk_size=32,
            out_dtype=torch.float32)
        assert torch.equal(o_n, out[a:b]), n
        assert torch.equal(f_n[0], fin[n]), n
    # A zero-length sequence hands its initial state through.
    assert torch.equal(fin[1], x.s0[1])


def test_shared_key_heads_equal_duplicated_heads():
    x = I.random_case(T_list=[90], h_k=2, h_v=4, d_k=32, d_v=32, io="f32",
                      seed=13, s0_std=0.05, device=DEV)
    out, fin = run_gpu(x, 32, False)
    qd = x.q.repeat_interleave(2, dim=1).contiguous()
    kd = x.k.repeat_interleave(2, dim=1).contiguous()
    out_d, fin_d = G.gdn_chunk_prefill(
        qd, kd, x.v, x.g, x.beta, x.A_log, x.dt_bias,
        initial_state=x.s0, chunk_size=32, out_dtype=torch.float32)
    assert torch.equal(out, out_d) and torch.equal(fin, fin_d)


def test_final_state_in_place():
    x = I.random_case(T_list=[50, 20], h_k=1, h_v=1, d_k=16, d_v=16, io="f32",
                      seed=17, s0_std=0.05, device=DEV)
    _, f_ref = run_oracle(x, False)
    st = x.s0.clone()
    G.gdn_chunk_prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                        cu_seqlens=x.cu_seqlens, initial_state=st,
                        final_state=st, chunk_size=16)
    assert per_state_rel(st, f_ref) <= TOL_F32_INPUTS


def test_direct_gates():
    x = I.random_case(T_list=[45], h_k=1, h_v=2, d_k=16, d_v=16, io="f32",
                      seed=19, s0_std=0.05, device=DEV)
    a = torch.rand(45, 2, device=DEV) * 0.5 + 0.5
    b = torch.rand(45, 2, device=DEV)
    out, fin = G.gdn_chunk_prefill(x.q, x.k, x.v, torch.log(a), b, None, None,
                                   initial_state=x.s0, chunk_size=16,
                                   gate_mode="direct", out_dtype=torch.float32)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, torch.log(a), b,
                             initial_state=x.s0, gate_mode="direct")
    assert per_head_rel(out, o_ref, [0, 45], 2, 16) <= TOL_F32_INPUTS
    assert per_state_rel(fin, f_ref) <= TOL_F32_INPUTS


def test_strong_decay_direct_gates():
    """fp32 path, chunk 16: direct log decays -30 u^3 with -200 (a decay of
    0 in fp32) on every 37th token, so e^G underflows inside a chunk and the
    state is wiped where a decay is 0."""
    T = 150
    x = I.random_case(T_list=[T], h_k=1, h_v=2, d_k=32, d_v=32, io="f32",
                      seed=43, s0_std=0.05, device=DEV)
    gen = torch.Generator().manual_seed(44)
    g = -30.0 * torch.rand(T, 2, generator=gen) ** 3
    g[9::37, 0] = -200.0
    g, b = g.to(DEV), torch.rand(T, 2, generator=gen).to(DEV)
    out, fin = G.gdn_chunk_prefill(x.q, x.k, x.v, g, b, None, None,
                                   initial_state=x.s0, chunk_size=16,
                                   gate_mode="direct", out_dtype=torch.float32)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, g, b, initial_state=x.s0,
                             gate_mode="direct")
    assert per_head_rel(out, o_ref, [0, T], 2, 32) <= TOL_F32_INPUTS
    assert per_state_rel(fin, f_ref) <= TOL_F32_INPUTS


def test_empty_prefill():
    x = I.random_case(T_list=[0, 0], h_k=1, h_v=1, d_k=16, d_v=16, io="f32",
                      seed=1, s0_std=0.05, device=DEV)
    out, fin = run_gpu(x, 16, False)
    assert out.numel() == 0 and torch.equal(fin, x.s0)
