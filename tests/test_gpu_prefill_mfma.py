"""GPU parity of the bf16 matrix-core prefill (bf16 inputs, d = 128, chunk
64) against the fp64 oracle, through the C ABI: the three prefill workloads
at full size (every head of the 4096-token layer; sampled (sequence, head)
chains of the 32768-token layer and of the packed 131048-token batch, each
run by the oracle over its whole length), and small cases with ragged chunk
tails, empty sequences, carried state, shared key heads, direct gates and
ill-conditioned keys."""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from parity import (TOL_BF16_INPUTS, bf16_ulp_diff, per_head_rel,
                    per_state_rel, rel_inf)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_prefill(x, tail, out_dtype=torch.float32, s0=True, **kw):
    return G.gdn_chunk_prefill(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
        cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_list,
        initial_state=x.s0 if s0 else None, z=x.z if tail else None,
        norm_weight=x.w, eps=x.eps, chunk_size=64, out_dtype=out_dtype, **kw)


def oracle_head(x, n, h, tail, group):
    """Oracle over the whole of sequence n, value head h."""
    a, b = x.cu_list[n], x.cu_list[n + 1]
    hk = h // group
    sl = lambda t, j: t[a:b, j:j + 1]
    s0 = None if x.s0 is None else x.s0[n:n + 1, h:h + 1]
    o, f = O.prefill(sl(x.q, hk), sl(x.k, hk), sl(x.v, h), sl(x.g, h),
                     sl(x.beta, h), x.A_log[h:h + 1], x.dt_bias[h:h + 1],
                     initial_state=s0)
    if tail:
        o = O.tail(o, sl(x.z, h), x.w, x.eps)
    return o.reshape(b - a, -1), f[0, 0]


def check_heads(x, out, fin, pairs, tail, group, label):
    d = x.v.shape[2]
    worst_o = worst_s = 0.0
    for (n, h) in pairs:
        a, b = x.cu_list[n], x.cu_list[n + 1]
        o_ref, f_ref = oracle_head(x, n, h, tail, group)
        o_gpu = out.reshape(out.shape[0], -1)[a:b, h * d:(h + 1) * d]
        e_o = rel_inf(o_gpu, o_ref) if b > a else 0.0
        e_s = rel_inf(fin[n, h], f_ref)
        print("%s seq %d head %d (len %d): out %.2e state %.2e"
              % (label, n, h, b - a, e_o, e_s))
        worst_o, worst_s = max(worst_o, e_o), max(worst_s, e_s)
    assert worst_o <= TOL_BF16_INPUTS, worst_o
    assert worst_s <= TOL_BF16_INPUTS, worst_s


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


def test_prefill_t32768_hv32_tail_sampled():
    """T=32768, 32 value / 16 key heads, fused tail: the slowest- and
    fastest-decaying heads, both value heads of one key head, and a middle
    head, each over the whole sequence; bf16 output == RNE(fp32 output)."""
    wl = I.WORKLOADS["prefill_t32768_hv32_tail"]
    x = I.make_inputs(wl, device=DEV)
    out, fin = gpu_prefill(x, True, s0=False)
    check_heads(x, out, fin, [(0, 0), (0, 14), (0, 15), (0, 31)], True, 2,
                "t32768")
    out16, fin16 = gpu_prefill(x, True, out_dtype=torch.bfloat16, s0=False)
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(fin16, fin)


def test_varlen_8seq_hv32_sampled():
    """8 packed sequences (131048 tokens) with carried initial states and the
    fused tail: the longest (65536) and the ragged (1000) sequences on two
    heads, plus the shortest on a third."""
    wl = I.WORKLOADS["varlen_8seq_hv32"]
    x = I.make_inputs(wl, device=DEV)
    out, fin = gpu_prefill(x, True)
    check_heads(x, out, fin, [(6, 3), (7, 3), (7, 30), (0, 17)], True, 2,
                "varlen")
    # Every final state moved away from its initial state and is finite.
    assert torch.isfinite(fin).all()
    assert torch.isfinite(out).all()


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
