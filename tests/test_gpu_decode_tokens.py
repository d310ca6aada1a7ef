"""GPU parity of gdn_decode_tokens (T decode tokens per sequence in one call,
optional per-token state snapshots) against the fp64 oracle, through the C
ABI: the outputs and final states equal the oracle's token-by-token
recurrence over each sequence's T tokens from its initial state, and every
snapshot equals the oracle state after that token."""
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


def _case(N, T, h_k, h_v, d, io, seed, tail=True, gates="spread"):
    return I.random_case(T_list=[T] * N, h_k=h_k, h_v=h_v, d_k=d, d_v=d,
                         io=io, seed=seed, gates=gates, tail=tail,
                         s0_std=0.05, device=DEV)


def _run(x, T, tail, snapshots=True, out_dtype=torch.float32, state=None):
    st = x.s0.clone() if state is None else state
    out, snaps = G.gdn_decode_tokens(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias, st, tokens_per_seq=T,
        snapshots=snapshots, z=x.z if tail else None, norm_weight=x.w,
        eps=x.eps, out_dtype=out_dtype)
    return out, snaps, st


def _oracle_snapshots(x, N, T, gate_mode="raw"):
    """State after each token, stepping the oracle's decode over token t of
    every sequence (rows n*T + t)."""
    st = x.s0
    snaps = []
    for t in range(T):
        rows = lambda a: a[t::T].contiguous()
        _, st = O.decode(rows(x.q), rows(x.k), rows(x.v), rows(x.g),
                         rows(x.beta), x.A_log, x.dt_bias, st,
                         gate_mode=gate_mode)
        snaps.append(st)
    return np.stack(snaps, axis=1)   # [N, T, h_v, d, d]


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("tail", [False, True])
@pytest.mark.parametrize("T", [1, 3, 8, 9, 20])
def test_tokens_small(d, io, tail, T):
    N, h_k, h_v = 4, 2, 4
    x = _case(N, T, h_k, h_v, d, io, seed=200 + d + T, tail=tail)
    out, snaps, st = _run(x, T, tail)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                             cu_seqlens=x.cu_list, initial_state=x.s0)
    if tail:
        o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    tol = TOL_F32_INPUTS if io == "f32" else TOL_BF16_INPUTS
    e_o = rel_inf(out.reshape(o_ref.shape), o_ref)
    e_s = per_state_rel(st, f_ref)
    s_ref = _oracle_snapshots(x, N, T)
    e_n = max(per_state_rel(snaps[:, t], s_ref[:, t]) for t in range(T))
    print("tokens d=%d io=%s tail=%d T=%d: out %.2e state %.2e snaps %.2e"
          % (d, io, tail, T, e_o, e_s, e_n))
    assert e_o <= tol and e_s <= tol and e_n <= tol
    # The last snapshot is the returned state.
    assert torch.equal(snaps[:, T - 1], st)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 20])
def test_tokens_strong_decay_direct_gates(io, T):
    """Log decays drawn down to -30 per token, some at -200 (a decay of 0 in
    fp32), as direct gates: the product of a batch's decays falls below
    2^-60 within a few tokens, so the kernel's rescaling of the rows it holds
    runs, on its own and after a token that wipes the state.  Outputs, final
    state and every snapshot against the oracle."""
    N, h_k, h_v, d = 4, 2, 4, 64
    x = _case(N, T, h_k, h_v, d, io, seed=31, tail=True)
    gen = torch.Generator().manual_seed(32)
    g = -30.0 * torch.rand(N * T, h_v, generator=gen)
    g[5::11, 1] = -200.0
    x.g = g.to(DEV)
    x.beta = torch.rand(N * T, h_v, generator=gen).to(DEV)
    st = x.s0.clone()
    out, snaps = G.gdn_decode_tokens(
        x.q, x.k, x.v, x.g, x.beta, None, None, st, tokens_per_seq=T,
        snapshots=True, z=x.z, norm_weight=x.w, eps=x.eps, gate_mode="direct",
        out_dtype=torch.float32)
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, None, None,
                             cu_seqlens=x.cu_list, initial_state=x.s0,
                             gate_mode="direct")
    o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    tol = TOL_F32_INPUTS if io == "f32" else TOL_BF16_INPUTS
    e_o = rel_inf(out.reshape(o_ref.shape), o_ref)
    e_s = per_state_rel(st, f_ref)
    s_ref = _oracle_snapshots(x, N, T, gate_mode="direct")
    e_n = max(per_state_rel(snaps[:, t], s_ref[:, t]) for t in range(T))
    print("tokens strong decay io=%s T=%d: out %.2e state %.2e snaps %.2e"
          % (io, T, e_o, e_s, e_n))
    assert e_o <= tol and e_s <= tol and e_n <= tol
    assert torch.equal(snaps[:, T - 1], st)


def test_tokens_full_size_speculative_batch():
    """256 sequences x 4 tokens, 32 value / 16 key heads, d = 128, bf16
    inputs, fused tail: every (token, head) output and every head's final
    state against the oracle; bf16 output == RNE of the fp32 output."""
    N, T = 256, 4
    x = _case(N, T, 16, 32, 128, "bf16", seed=11, tail=True)
    out, snaps, st = _run(x, T, True, snapshots=False)
    assert snaps is None
    o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                             cu_seqlens=x.cu_list, initial_state=x.s0)
    o_ref = O.tail(o_ref, x.z, x.w, x.eps)
    e_o = rowwise_rel(out, o_ref, 128)
    e_s = rowwise_rel(st, f_ref, 128 * 128)
    print("tokens full: out %.2e state %.2e" % (e_o, e_s))
    assert e_o <= TOL_BF16_INPUTS and e_s <= TOL_BF16_INPUTS
    out16, _, st16 = _run(x, T, True, snapshots=False, out_dtype=torch.bfloat16)
    assert bf16_ulp_diff(out16, out) <= 1
    assert torch.equal(st16, st)


def test_tokens_full_size_snapshots():
    """256 sequences x 4 tokens, 32 value / 16 key heads, d = 128, bf16,
    tail, snapshots on (2 GiB of them): outputs and final state equal the
    call without snapshots bit for bit; snapshot 3 is the returned state;
    snapshots 1 and 2 equal the final states of calls over the first 2 and
    3 tokens of each sequence; snapshot 0 of every head against the
    oracle's decode step."""
    N, T = 256, 4
    x = _case(N, T, 16, 32, 128, "bf16", seed=13, tail=True)
    out, snaps, st = _run(x, T, True, snapshots=True)
    out_n, _, st_n = _run(x, T, True, snapshots=False)
    assert torch.equal(out, out_n) and torch.equal(st, st_n)
    assert torch.equal(snaps[:, T - 1], st)
    for t in (1, 2):
        keep = t + 1
        sub = lambda a: torch.stack([a[n * T:n * T + keep] for n in range(N)]
                                    ).reshape(N * keep, *a.shape[1:]).contiguous()
        st_t = x.s0.clone()
        G.gdn_decode_tokens(sub(x.q), sub(x.k), sub(x.v), sub(x.g), sub(x.beta),
                            x.A_log, x.dt_bias, st_t, tokens_per_seq=keep,
                            z=sub(x.z), norm_weight=x.w, eps=x.eps,
                            out_dtype=torch.float32)
        assert torch.equal(snaps[:, t], st_t), t
    rows = lambda a: a[0::T].contiguous()
    _, s_ref = O.decode(rows(x.q), rows(x.k), rows(x.v), rows(x.g),
                        rows(x.beta), x.A_log, x.dt_bias, x.s0)
    e_0 = rowwise_rel(snaps[:, 0].contiguous(), s_ref, 128 * 128)
    print("tokens full snapshots: snapshot 0 %.2e" % e_0)
    assert e_0 <= TOL_BF16_INPUTS


def test_tokens_one_equals_decode_step():
    x = _case(6, 1, 2, 4, 128, "bf16", seed=5, tail=True)
    out_t, _, st_t = _run(x, 1, True, snapshots=False)
    st_d = x.s0.clone()
    out_d = G.gdn_decode_step(x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
                              st_d, z=x.z, norm_weight=x.w, eps=x.eps,
                              out_dtype=torch.float32)
    assert torch.equal(out_t, out_d) and torch.equal(st_t, st_d)


def test_tokens_resume_from_snapshot():
    """Rolling back to the snapshot after token 1 and re-running tokens 2..T-1
    from it reproduces the full call exactly (what a speculative decoder does
    after rejecting drafts)."""
    N, T = 3, 5
    x = _case(N, T, 1, 2, 64, "bf16", seed=9, tail=True)
    out, snaps, st = _run(x, T, True)
    keep = 2
    resume = snaps[:, keep - 1].contiguous()
    sub = lambda a: torch.stack([a[n * T + keep:(n + 1) * T]
                                 for n in range(N)]).reshape(
                                     N * (T - keep), *a.shape[1:]).contiguous()
    out2, _ = G.gdn_decode_tokens(
        sub(x.q), sub(x.k), sub(x.v), sub(x.g), sub(x.beta), x.A_log,
        x.dt_bias, resume, tokens_per_seq=T - keep, z=sub(x.z),
        norm_weight=x.w, eps=x.eps, out_dtype=torch.float32)
    assert torch.equal(resume, st)
    assert torch.equal(out2, sub(out))


def test_tokens_empty():
    x = _case(2, 2, 1, 1, 16, "f32", seed=1, tail=False)
    st = x.s0.clone()
    out, snaps = G.gdn_decode_tokens(x.q[:0], x.k[:0], x.v[:0], x.g[:0],
                                     x.beta[:0], x.A_log, x.dt_bias, st,
                                     tokens_per_seq=0, snapshots=True)
    assert out.numel() == 0 and snaps.numel() == 0
    assert torch.equal(st, x.s0)
