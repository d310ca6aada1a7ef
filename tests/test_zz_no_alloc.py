"""gdn_chunk_prefill_noalloc (the prefill on the library's static per-GPU
scratch) against gdn_chunk_prefill (caller's workspace) through the C ABI:
the same kernels run on the same inputs, so outputs and final states must be
identical.  Two calls in a row, the second smaller, show that the scratch
keeps no state a later call depends on.  Both are checked against the
oracle too."""
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import binding as B
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from parity import TOL_BF16_INPUTS, per_head_rel, per_state_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(x, tail, out_dtype, label):
    ref_out, ref_fin = G.gdn_chunk_prefill(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
        cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_list,
        initial_state=x.s0, z=x.z if tail else None, norm_weight=x.w,
        eps=x.eps, chunk_size=64, out_dtype=out_dtype)
    out = torch.full_like(ref_out, float("nan"))
    fin = torch.full_like(ref_fin, float("nan"))
    args, keep = B.make_prefill_args(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias,
        cu_seqlens=x.cu_seqlens, num_seqs=len(x.cu_list) - 1,
        initial_state=x.s0, final_state=fin, z=x.z if tail else None,
        norm_weight=x.w, eps=x.eps, chunk_size=64, out=out,
        out_dtype=B._dt(out))
    need = B.gdn_prefill_workspace_size(args)
    del keep
    assert 0 < need <= B.NOALLOC_SCRATCH_BYTES, (label, need)
    print("noalloc %s call: T=%d seqs=%d h_v=%d tail=%s workspace %d bytes"
          % (label, x.q.shape[0], len(x.cu_list) - 1, x.v.shape[1], tail,
             need), flush=True)
    G.gdn_chunk_prefill_noalloc(
        x.q, x.k, x.v, x.g, x.beta, x.A_log, x.dt_bias, out=out,
        cu_seqlens=x.cu_seqlens, cu_seqlens_host=x.cu_list,
        initial_state=x.s0, final_state=fin, z=x.z if tail else None,
        norm_weight=x.w, eps=x.eps, chunk_size=64)
    torch.cuda.synchronize()
    return ref_out, ref_fin, out, fin


def test_noalloc_prefill_matches_workspace_prefill_twice():
    # First call: three sequences (ragged chunk tails) with carried state,
    # 8 value heads over 4 key heads, gated tail, bf16 output.
    a = I.random_case(T_list=[1500, 64, 2033], h_k=4, h_v=8, d_k=128, d_v=128,
                      seed=11, tail=True, s0_std=0.05, device=DEV)
    # Second call, smaller: one 700-token sequence, no tail, fp32 output.
    b = I.random_case(T_list=[700], h_k=2, h_v=4, d_k=128, d_v=128, seed=12,
                      device=DEV)
    for x, tail, odt, label in ((a, True, torch.bfloat16, "first"),
                                (b, False, torch.float32, "second")):
        ref_out, ref_fin, out, fin = _pair(x, tail, odt, label)
        assert torch.equal(out, ref_out), label
        assert torch.equal(fin, ref_fin), label
        o_ref, f_ref = O.prefill(x.q, x.k, x.v, x.g, x.beta, x.A_log,
                                 x.dt_bias, cu_seqlens=x.cu_list,
                                 initial_state=x.s0)
        assert per_state_rel(fin, f_ref) <= TOL_BF16_INPUTS, label
        if not tail:
            assert per_head_rel(out, o_ref, x.cu_list, x.v.shape[1],
                                128) <= TOL_BF16_INPUTS, label
