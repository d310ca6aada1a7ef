"""GPU parity of gdn_out_proj (the ssm_out projection after the gated tail,
dense bf16 or packed Q4_K weight decoded on the GPU) against the fp64 Q4_K
oracle, through the C ABI.  Errors are per token row: max |y - ref| /
max |ref| over the row's out features."""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import oracle as O
from oracle import q4k as Q
from parity import TOL_BF16_INPUTS, TOL_F32_INPUTS, bf16_ulp_diff, rowwise_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _x(M, K, io, seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    return torch.randn(M, K, generator=gen, device=DEV).to(dt)


def _weight(fmt, N, K, seed):
    if fmt == "q4k":
        return I.q4k_weight(N, K, seed=seed, subnormal_rows=1, device=DEV)
    return I.dense_weight(N, K, seed=seed, device=DEV)


def _ref(x, w, fmt, N, Wdec=None):
    if fmt == "q4k":
        if Wdec is None:
            return Q.project(x, w, N)
        return Q.project_dense(x, Wdec)
    return Q.project_dense(x, w)


def _tol(io):
    return TOL_BF16_INPUTS if io == "bf16" else TOL_F32_INPUTS


@pytest.mark.parametrize("fmt", ["q4k", "bf16"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N", [
    (1, 256, 64),        # matrix-vector kernel, one block per row
    (3, 512, 68),        # matrix-vector, ragged out rows
    (8, 4096, 2048),     # matrix-vector at the layer's shape, 8 tokens
    (9, 256, 64),        # smallest tile-kernel case
    (37, 512, 132),      # ragged tokens and out rows, 32 x 64 tiles, K split
    (1500, 512, 260),    # 64 x 64 tiles, K split in 2, ragged both ways
    (5000, 512, 260),    # above 4096 tokens: the GEMM (bf16 x), 128 x 128 or 64 x 64 tiles (fp32 x)
])
def test_out_proj_small(fmt, io, M, K, N):
    x = _x(M, K, io, seed=M + K + N)
    w = _weight(fmt, N, K, seed=N)
    y = G.gdn_out_proj(x, w, N, q4k=fmt == "q4k", out_dtype=torch.float32)
    ref = _ref(x, w, fmt, N)
    e = rowwise_rel(y, ref, N)
    y16 = G.gdn_out_proj(x, w, N, q4k=fmt == "q4k", out_dtype=torch.bfloat16)
    u = bf16_ulp_diff(y16, y)
    print("out_proj %s io=%s M=%d K=%d N=%d: %.2e (bf16 out %d ulp)"
          % (fmt, io, M, K, N, e, u))
    assert e <= _tol(io) and u <= 1


@pytest.mark.parametrize("fmt,M,K,N", [
    ("bf16", 4097, 64, 4),       # one K step, one out-row tile of 4 rows
    ("bf16", 4097, 128, 1028),   # two K steps, ragged out-row tile
    ("q4k", 4097, 256, 4),       # one Q4_K block per row: 8 steps over both parts
    ("q4k", 4097, 512, 1028),
])
def test_out_proj_large_m_edges(fmt, M, K, N):
    """Dense bf16 and decoded Q4_K above 4096 tokens (the direct-to-LDS
    GEMM): few K steps (the loads issued past the last step), ragged token
    and out-row tiles; every row against the oracle."""
    x = _x(M, K, "bf16", seed=M + K)
    w = _weight(fmt, N, K, seed=N)
    y = G.gdn_out_proj(x, w, N, q4k=fmt == "q4k", out_dtype=torch.float32)
    e = rowwise_rel(y, _ref(x, w, fmt, N), N)
    y16 = G.gdn_out_proj(x, w, N, q4k=fmt == "q4k", out_dtype=torch.bfloat16)
    u = bf16_ulp_diff(y16, y)
    print("out_proj %s M=%d K=%d N=%d: %.2e (bf16 out %d ulp)" % (fmt, M, K, N, e, u))
    assert e <= TOL_BF16_INPUTS and u <= 1


@pytest.mark.parametrize("fmt", ["q4k", "bf16"])
def test_out_proj_layer_shapes(fmt):
    """The layer's projection (4096 -> 2048) at the decode batch (256 tokens)
    and at the 32768-token prefill, bf16 activations: all 256 decode rows and
    384 sampled prefill rows (first, last, random) against the oracle; the
    bf16 output within one ulp of the fp32 output."""
    K, N = 4096, 2048
    w = _weight(fmt, N, K, seed=5)
    Wdec = Q.decode_matrix(w.cpu().numpy(), N, K) if fmt == "q4k" else None
    for M, nsample in ((256, 256), (32768, 384)):
        x = _x(M, K, "bf16", seed=M)
        y = G.gdn_out_proj(x, w, N, q4k=fmt == "q4k", out_dtype=torch.float32)
        y16 = G.gdn_out_proj(x, w, N, q4k=fmt == "q4k")
        rng = np.random.default_rng(M)
        rows = np.unique(np.concatenate([
            [0, M - 1], rng.choice(M, min(M, nsample), replace=False)]))
        idx = torch.as_tensor(rows, device=DEV)
        ref = _ref(x[idx], w, fmt, N, Wdec)
        e = rowwise_rel(y[idx], ref, N)
        u = bf16_ulp_diff(y16, y)
        print("out_proj %s M=%d: %.2e over %d rows (bf16 out %d ulp)"
              % (fmt, M, e, rows.size, u))
        assert e <= TOL_BF16_INPUTS and u <= 1


def test_field_gate_one_token():
    """One token through the tail and the Q4_K projection at the layer's
    shapes (32 value heads x 128 -> 4096 -> 2048): every one of the 4096
    gated-normalized values and every one of the 2048 projected outputs
    against the oracle."""
    h_v, d = 32, 128
    gen = torch.Generator(device=DEV).manual_seed(77)
    o = torch.randn(1, h_v, d, generator=gen, device=DEV)
    z = torch.randn(1, h_v, d, generator=gen, device=DEV)
    nw = 0.5 + torch.rand(d, generator=gen, device=DEV)
    w = I.q4k_weight(2048, 4096, seed=78, device=DEV)
    gated = G.gdn_gated_rmsnorm(o, z, nw, 1e-6)
    ref_g = O.gated_rmsnorm(o, z, nw, 1e-6).reshape(1, 4096)
    y = G.gdn_out_proj(gated.reshape(1, 4096), w, 2048, q4k=True)
    ref_y = Q.project(gated.reshape(1, 4096), w, 2048)
    e_g = rowwise_rel(gated.reshape(1, 4096), ref_g, 4096)
    e_y = rowwise_rel(y, ref_y, 2048)
    print("field gate: gated %.2e projected %.2e" % (e_g, e_y))
    assert e_g <= TOL_F32_INPUTS and e_y <= TOL_F32_INPUTS


def test_out_proj_deterministic_and_empty():
    """Split-K partial sums are added in a fixed order: repeated calls give
    identical bits; a reused, dirty workspace changes nothing."""
    x = _x(300, 512, "bf16", seed=1)
    w = _weight("q4k", 128, 512, seed=2)
    a = G.gdn_out_proj(x, w, 128, q4k=True)
    ws = torch.full((1 << 22,), 255, dtype=torch.uint8, device=DEV)
    b = G.gdn_out_proj(x, w, 128, q4k=True, workspace=ws)
    c = G.gdn_out_proj(x, w, 128, q4k=True, workspace=ws)
    assert torch.equal(a, b) and torch.equal(b, c)
    y = G.gdn_out_proj(x[:0], w, 128, q4k=True)
    assert y.shape == (0, 128)


def test_out_proj_rejects_bad_shapes():
    x = _x(4, 300, "bf16", seed=1)
    w = torch.zeros(64, 300, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError):
        G.gdn_out_proj(x, w, 64)
