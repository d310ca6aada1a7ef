"""GPU parity of the bf16 matrix-core prefill (bf16 inputs, d = 128, chunk
64) against the fp64 oracle, through the C ABI: the three prefill workloads
at full size (every head and every value of the 4096-token layer, the
32768-token layer and all 8 x 32 chains of the packed 131048-token batch,
each chain run by the oracle over its whole length), and small cases with ragged chunk
tails, empty sequences, carried state, shared key heads, direct gates and
ill-conditioned keys."""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from parity import (TOL_BF16_INPUTS, bf16_ulp_diff, per_head_rel,
                    per_state_rel, rel_inf, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_prefill(x, tail, out_dtype=torch.float32, s0=True, **kw):
    return G.gdn_chunk_prefill(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
        cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_list,
        initial_state=x.s0 if s0 else None, z=x.z if tail else None,
        norm_weight=x.w, eps=x.eps, chunk_size=64, out_dtype=out_dtype, **kw)


def test_prefill_t4096_h8_all_heads():
    """B=1, T=4096, 8 heads, d=128, bf16, chunk 64, zero initial state:
    every output and the whole final state against the oracle."""
    wl = I.WORKLOADS["prefill_t4096_h8"]
    x = I.make_inputs(wl, device=DEV)
    out, fin = gpu_prefill(x, False, s0=False)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias)
    e_o = per_head_rel(out, o_ref, x.cu_list, 8, 128)
    e_s = per_state_rel(fin, f_ref)
    print("t4096: out %.2e state %.2e" % (e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS
    out16, fin16 = gpu_prefill(x, False, out_dtype=torch.bfloat16, s0=False)
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(fin16, fin)


def check_all_chains(x, out, fin, tail, label):
    """Every (sequence, value head) chain against the oracle over its whole
    length: the fp32-mode output and the final state, each at the bf16-input
    tolerance.  The oracle runs one sequence at a time (all its heads in one
    call) to bound host memory."""
    h_v, d = x.v.shape[1], x.v.shape[2]
    worst_o = worst_s = 0.0
    for n in range(len(x.cu_list) - 1):
        a, b = x.cu_list[n], x.cu_list[n + 1]
        s0 = None if x.s0 is None else x.s0[n:n + 1]
        o_ref, f_ref = O.prefill(x.q[a:b], x.k[a:b], x.v[a:b], x.g[a:b],
                                 x.beta[a:b], x.A_log, x.dt_bias,
                                 initial_state=s0)
        if tail:
            o_ref = O.tail(o_ref, x.z[a:b], x.w, x.eps)
        o_ref = o_ref.reshape(b - a, h_v, d)
        o_gpu = to_np(out[a:b]).reshape(b - a, h_v, d)
        f_gpu = to_np(fin[n])
        seq_o = max((rel_inf(o_gpu[:, h], o_ref[:, h]) for h in range(h_v)),
                    default=0.0) if b > a else 0.0
        seq_s = max(rel_inf(f_gpu[h], f_ref[0, h]) for h in range(h_v))
        print("%s seq %d (len %d), all %d heads: out %.2e state %.2e"
              % (label, n, b - a, h_v, seq_o, seq_s))
        worst_o, worst_s = max(worst_o, seq_o), max(worst_s, seq_s)
        del o_ref, o_gpu
    assert worst_o <= TOL_BF16_INPUTS, worst_o
    assert worst_s <= TOL_BF16_INPUTS, worst_s


def test_prefill_t32768_hv32_tail_all_heads():
    """T=32768, 32 value / 16 key heads, fused tail: every output value and
    the whole final state of all 32 heads against the oracle; the bf16
    output is RNE(fp32 output) within one ulp."""
    wl = I.WORKLOADS["prefill_t32768_hv32_tail"]
    x = I.make_inputs(wl, device=DEV)
    out, fin = gpu_prefill(x, True, s0=False)
    check_all_chains(x, out, fin, True, "t32768")
    out16, fin16 = gpu_prefill(x, True, out_dtype=torch.bfloat16, s0=False)
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(fin16, fin)


def test_varlen_8seq_hv32_all_chains():
    """8 packed sequences (131048 tokens) with carried initial states and the
    fused tail: all 8 x 32 (sequence, head) chains, outputs and final
    states, against the oracle; every final state has moved away from its
    initial state; the bf16 output is RNE(fp32 output) within one ulp."""
    wl = I.WORKLOADS["varlen_8seq_hv32"]
    x = I.make_inputs(wl, device=DEV)
    out, fin = gpu_prefill(x, True)
    check_all_chains(x, out, fin, True, "varlen")
    moved = (fin - x.s0).abs().amax(dim=(2, 3)) / x.s0.abs().amax(dim=(2, 3))
    assert bool((moved > 0.1).all()), float(moved.min())
    out16, fin16 = gpu_prefill(x, True, out_dtype=torch.bfloat16)
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(fin16, fin)


SMALL = [
    # lens, h_k, h_v, tail, s0, gates
    ([1], 1, 1, False, False, "spread"),
    ([15, 16, 17], 1, 2, True, True, "spread"),
    ([63, 64, 65], 2, 2, False, True, "tiny"),
    ([200, 0, 129], 2, 4, True, True, "spread"),
    ([0, 0], 1, 1, False, True, "spread"),
    ([1000], 1, 2, True, True, "tiny"),
    # 2, 3, 5 and 6 chunks: every way the scan's chunk pairs can end
    ([128, 192, 257, 384], 1, 2, True, True, "spread"),
    # four value heads per key head (K and Q fragments written by heads 0, 1)
    ([300, 5], 1, 4, True, True, "spread"),
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_small_cases(case):
    lens, h_k, h_v, tail, s0, gates = case
    x = I.random_case(T_list=lens, h_k=h_k, h_v=h_v, d_k=128, d_v=128,
                      io="bf16", seed=31 + sum(lens), gates=gates, tail=tail,
                      s0_std=0.05 if s0 else None, device=DEV)
    out, fin = gpu_prefill(x, tail, s0=s0)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                             cu_seqlens=x.cu_list,
                             initial_state=x.s0 if s0 else None)
    if tail:
        o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    e_o = per_head_rel(out, o_ref, x.cu_list, h_v, 128)
    e_s = per_state_rel(fin, f_ref)
    print("small %s: out %.2e state %.2e" % (case, e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS


def _strong_decays(T, h_v, seed):
    """Direct log decays -30 u^3 (u uniform: most near 0, a tail down to
    -30), and -200 (a decay of 0 in fp32) on every 37th token of head 0."""
    gen = torch.Generator().manual_seed(seed)
    g = -30.0 * torch.rand(T, h_v, generator=gen) ** 3
    g[9::37, 0] = -200.0
    return g.to(DEV), torch.rand(T, h_v, generator=gen).to(DEV)


def test_strong_decay_direct_gates():
    """Chunk-local sums of the log decays reach -300 to -900, so
    e^G underflows to 0 inside a chunk, and a decay of 0 wipes the state:
    the path must form every e^(G_i - G_j) from the difference.  Packed
    sequences with the tail and an initial state; outputs and final states
    against the oracle."""
    lens = [200, 77]
    x = I.random_case(T_list=lens, h_k=1, h_v=2, d_k=128, d_v=128, io="bf16",
                      seed=41, tail=True, s0_std=0.05, device=DEV)
    x.g, x.beta = _strong_decays(sum(lens), 2, 42)
    out, fin = G.gdn_chunk_prefill(
        x.q, x.k, x.v, x.g, x.beta, None, None, cu_seqlens=x.cu_seqlens,
        cu_seqlens_host=x.cu_list, initial_state=x.s0, z=x.z, norm_weight=x.w,
        eps=x.eps, chunk_size=64, gate_mode="direct", out_dtype=torch.float32)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, None, None,
                             cu_seqlens=x.cu_list, initial_state=x.s0,
                             gate_mode="direct")
    o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    e_o = per_head_rel(out, o_ref, x.cu_list, 2, 128)
    e_s = per_state_rel(fin, f_ref)
    print("strong decay: out %.2e state %.2e" % (e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS


def test_final_state_in_place():
    """final_state == initial_state (allowed by the header) on the matrix-
    core path: packed sequences, one empty, with the tail; equals the call
    with separate buffers bit for bit."""
    lens = [200, 0, 129, 64]
    x = I.random_case(T_list=lens, h_k=2, h_v=4, d_k=128, d_v=128, io="bf16",
                      seed=47, tail=True, s0_std=0.05, device=DEV)
    out, fin = gpu_prefill(x, True)
    st = x.s0.clone()
    out2, fin2 = G.gdn_chunk_prefill(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias, cu_seqlens=x.cu_seqlens,
        cu_seqlens_host=x.cu_list, initial_state=st, final_state=st, z=x.z,
        norm_weight=x.w, eps=x.eps, chunk_size=64, out_dtype=torch.float32)
    assert fin2.data_ptr() == st.data_ptr()
    assert torch.equal(out2, out) and torch.equal(st, fin)


def test_many_groups_per_team_with_tail():
    """96 sequences of 0..400 tokens, 2 value heads each: more (sequence,
    head) groups than the gated scan's persistent teams, so every team walks
    several groups of mixed lengths (including ones shorter than the tail's
    lag) with the cross-slice exchange; every head against the oracle, and
    the bf16 output within one ulp of the fp32 one."""
    gen = np.random.default_rng(8)
    lens = [int(v) for v in gen.integers(0, 401, size=96)]
    lens[3] = 0
    lens[7] = 1
    x = I.random_case(T_list=lens, h_k=1, h_v=2, d_k=128, d_v=128, io="bf16",
                      seed=91, tail=True, s0_std=0.05, device=DEV)
    out, fin = gpu_prefill(x, True)
    out16, fin16 = gpu_prefill(x, True, out_dtype=torch.bfloat16)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                             cu_seqlens=x.cu_list, initial_state=x.s0)
    o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    e_o = per_head_rel(out, o_ref, x.cu_list, 2, 128)
    e_s = per_state_rel(fin, f_ref)
    print("many groups: out %.2e state %.2e" % (e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(fin16, fin)


def test_ill_conditioned_keys_and_full_writes():
    """Runs of identical keys with write strength near 1 and no decay stress
    the UT inverse; direct gates; compared with the oracle."""
    T = 192
    gen = torch.Generator(device=DEV).manual_seed(5)
    base = torch.randn(8, 128, generator=gen, device=DEV)
    k = base.repeat_interleave(24, dim=0)[:T]
    k = k + 1e-3 * torch.randn(T, 128, generator=gen, device=DEV)
    k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)[:, None]
    q = torch.randn(T, 1, 128, generator=gen, device=DEV)
    q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    v = torch.randn(T, 1, 128, generator=gen, device=DEV).to(torch.bfloat16)
    g = torch.full((T, 1), -1e-4, device=DEV)
    b = torch.full((T, 1), 0.999, device=DEV)
    out, fin = G.gdn_chunk_prefill(q, k, v, g, b, None, None, chunk_size=64,
                                   gate_mode="direct", out_dtype=torch.float32)
    o_ref, f_ref = O.prefill(q, k, v, g, b, gate_mode="direct")
    e_o, e_s = rel_inf(out, o_ref), rel_inf(fin[0, 0], f_ref[0, 0])
    print("ill-conditioned: out %.2e state %.2e" % (e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS


def test_packed_equals_separate_split_and_deterministic():
    lens = [130, 0, 64, 300]
    x = I.random_case(T_list=lens, h_k=2, h_v=4, d_k=128, d_v=128, io="bf16",
                      seed=77, tail=True, s0_std=0.05, device=DEV)
    out, fin = gpu_prefill(x, True)
    out2, fin2 = gpu_prefill(x, True)
    assert torch.equal(out, out2) and torch.equal(fin, fin2)
    cu = x.cu_list
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = lambda t: t[a:b].contiguous()
        o_n, f_n = G.gdn_chunk_prefill(
            sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.A_log,
            x.dt_bias, initial_state=x.s0[n:n + 1].contiguous(), z=sl(x.z),
            norm_weight=x.w, eps=x.eps, chunk_size=64,
            out_dtype=torch.float32)
        assert torch.equal(o_n, out[a:b]), n
        assert torch.equal(f_n[0], fin[n]), n
    # Split at a chunk boundary: the carried state continues exactly.
    a, b = cu[3], cu[4]
    sl = lambda t, u, v_: t[u:v_].contiguous()
    _, f1 = G.gdn_chunk_prefill(sl(x.q, a, a + 128), sl(x.k, a, a + 128),
                                sl(x.v, a, a + 128), sl(x.g, a, a + 128),
                                sl(x.beta, a, a + 128), x.A_log, x.dt_bias,
                                initial_state=x.s0[3:4].contiguous(),
                                chunk_size=64)
    _, f2 = G.gdn_chunk_prefill(sl(x.q, a + 128, b), sl(x.k, a + 128, b),
                                sl(x.v, a + 128, b), sl(x.g, a + 128, b),
                                sl(x.beta, a + 128, b), x.A_log, x.dt_bias,
                                initial_state=f1, chunk_size=64)
    assert torch.equal(f2[0], fin[3])


def test_shared_key_heads_equal_duplicated():
    x = I.random_case(T_list=[150], h_k=2, h_v=4, d_k=128, d_v=128,
                      io="bf16", seed=3, s0_std=0.05, device=DEV)
    out, fin = gpu_prefill(x, False)
    qd = x.q.repeat_interleave(2, dim=1).contiguous()
    kd = x.k.repeat_interleave(2, dim=1).contiguous()
    out_d, fin_d = G.gdn_chunk_prefill(qd, kd, x.v, x.g, x.beta, x.A_log,
                                       x.dt_bias, initial_state=x.s0,
                                       chunk_size=64, out_dtype=torch.float32)
    assert torch.equal(out, out_d) and torch.equal(fin, fin_d)
