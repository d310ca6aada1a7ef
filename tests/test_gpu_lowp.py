"""GPU parity of the low-precision projections (W8A8 FP8 and W4A4 MXFP4)
and of their activation quantizer, through the C ABI, against the fp64
oracle (oracle/lowp.py).

* Quantized codes and scales are integers decided on the same exact values
  on both sides (divisions by powers of two), so they must match bit for
  bit.
* The projection multiplies those codes; the matrix cores form exact
  products and add them in fp32, so the bound is the one of an fp32 dot
  product of K terms: |y - ref| <= K 2^-24 sum_k |x_k w_k| (fp32 output),
  ref being the exact fp64 product of the dequantized codes.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrence_delta_amd as G
from gated_deltanet_recurrence_delta_amd import inputs as I
from oracle import lowp as L
from parity import bf16_ulp_diff

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _x(M, K, io, seed, spread=True):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(M, K, generator=gen, device=DEV)
    if spread:       # rows of very different magnitudes, a zero row
        mag = 10.0 ** torch.randint(-6, 7, (M, 1), generator=gen, device=DEV)
        x = x * mag
        if M > 2:
            x[1] = 0.0
    return x.to(torch.bfloat16 if io == "bf16" else torch.float32)


def _ties_x(K, io):
    """A row whose values sit exactly on E4M3 and E2M1 rounding ties."""
    ties = [0.5 * (a + b) for a, b in ((1.0, 1.125), (2.0, 2.25), (0.25, 0.28125),
                                       (1.5, 1.625), (448 - 16, 448))]
    v = np.resize(np.array(ties + [-t for t in ties] + [2.5, 5.0, 0.75, 0.25, 1.25, 1.75, 3.5]), K)
    v[0] = 448.0
    return torch.tensor(v[None, :], dtype=torch.float32, device=DEV).to(
        torch.bfloat16 if io == "bf16" else torch.float32)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_quantizer_bit_exact(fmt, io):
    # 4224 values per row exceed what one wave holds in registers and take
    # the two-pass FP8 kernel.
    for x in (_x(37, 512, io, seed=5), _x(6, 4096, io, seed=6), _ties_x(256, io),
              _x(3, 4224 if fmt == "fp8" else 4352, io, seed=7)):
        codes, scales = G.gdn_quantize_act(x, fmt)
        if fmt == "fp8":
            rc, re = L.quantize_rows_fp8(x.float().cpu().numpy())
            assert np.array_equal(codes.cpu().numpy(), rc)
            assert np.array_equal(scales.cpu().double().numpy(), 2.0 ** re)
        else:
            rc, rs = L.quantize_rows_mxfp4(x.float().cpu().numpy())
            assert np.array_equal(codes.cpu().numpy(), L.pack_fp4(rc))
            assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_quantizer_signed_zeros(fmt, io):
    """Exact zeros of both signs -- scattered in nonzero rows, filling whole
    32-value blocks, and making up a whole row -- quantize as the oracle's
    encoders read them (E4M3 keeps a zero's sign; an exact zero's E2M1 code
    is the positive one)."""
    x = _x(4, 512, io, seed=11)
    neg0 = torch.tensor(-0.0, dtype=x.dtype, device=x.device)
    x[0, ::3] = 0.0
    x[1, 1::4] = neg0
    x[2, :64] = neg0
    x[3, :] = 0.0
    x[3, 5::7] = neg0
    assert bool(torch.signbit(x[1, 1]).item()) and not bool(torch.signbit(x[0, 0]).item())
    codes, scales = G.gdn_quantize_act(x, fmt)
    if fmt == "fp8":
        rc, re = L.quantize_rows_fp8(x.float().cpu().numpy())
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert np.array_equal(scales.cpu().double().numpy(), 2.0 ** re)
    else:
        rc, rs = L.quantize_rows_mxfp4(x.float().cpu().numpy())
        assert np.array_equal(codes.cpu().numpy(), L.pack_fp4(rc))
        assert np.array_equal(scales.cpu().numpy(), rs)


def test_mxfp4_quantizer_large_input_bit_exact():
    """2^19 blocks take the one-thread-per-block kernel; sampled rows are
    checked bit for bit."""
    x = _x(2048, 8192, "bf16", seed=9)
    codes, scales = G.gdn_quantize_act(x, "mxfp4")
    rows = [0, 1, 777, 2047]
    rc, rs = L.quantize_rows_mxfp4(x[rows].float().cpu().numpy())
    assert np.array_equal(codes[rows].cpu().numpy(), L.pack_fp4(rc))
    assert np.array_equal(scales[rows].cpu().numpy(), rs)


def _weights(fmt, N, K, seed):
    if fmt == "fp8":
        return I.fp8_weight(N, K, seed=seed, device=DEV)
    return I.mxfp4_weight(N, K, seed=seed, device=DEV)


def _reference(fmt, x, w, ws):
    xn = x.float().cpu().numpy()
    if fmt == "fp8":
        y, xc, xe = L.project_fp8(xn, w.cpu().numpy(), ws.cpu().numpy())
        X = L.dequant_fp8(xc, 2.0 ** xe.astype(float))
        W = L.dequant_fp8(w.cpu().numpy(), ws.cpu().double().numpy())
    else:
        y, xp, xs = L.project_mxfp4(xn, w.cpu().numpy(), ws.cpu().numpy())
        X = L.dequant_mxfp4(L.unpack_fp4(xp), xs)
        W = L.dequant_mxfp4(L.unpack_fp4(w.cpu().numpy()), ws.cpu().numpy())
    return y, L.abs_product(X, W)


def _check(fmt, x, w, ws, N, rows=None):
    y = G.gdn_out_proj(x, w, N, weight_format=fmt, weight_scale=ws,
                       out_dtype=torch.float32)
    y16 = G.gdn_out_proj(x, w, N, weight_format=fmt, weight_scale=ws,
                         out_dtype=torch.bfloat16)
    xs = x if rows is None else x[torch.as_tensor(rows, device=DEV)]
    ys = y if rows is None else y[torch.as_tensor(rows, device=DEV)]
    ref, absprod = _reference(fmt, xs, w, ws)
    K = x.shape[1]
    err = np.abs(ys.cpu().double().numpy() - ref)
    # Exact products of codes and fp32 accumulation across instructions
    # (K 2^-24), plus each 128-value instruction's own block sum, which is not
    # sequential fp32: up to 2^-14.3 of the block's sum |x w| measured on
    # full-range codes, allowed 2^-13 (summed over the blocks).
    bound = (K * 2.0 ** -24 + 2.0 ** -13) * absprod + 1e-30
    ratio = float(np.max(err / bound))
    # Independently of that fitted bound, every row meets the path's
    # tolerance for bf16-input products: max |y - ref| / max |ref| <= 2e-3
    # (rows whose exact product is all zero must come out exactly zero).
    den = np.max(np.abs(ref), axis=1)
    num = np.max(err, axis=1)
    assert np.all(num[den == 0] == 0)
    row_rel = float(np.max(num[den > 0] / den[den > 0])) if np.any(den > 0) else 0.0
    assert row_rel <= 2e-3, row_rel
    return ratio, bf16_ulp_diff(y16, y)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N", [
    (1, 512, 64), (9, 512, 64), (37, 1024, 132), (300, 512, 128),
    (1500, 512, 260), (5000, 512, 260),
    # above 4096 tokens (256 x 256 tiles): one MXFP4 step (two FP8 steps),
    # ragged token and out-row tiles
    (4097, 256, 4), (4097, 512, 1028)])
def test_lowp_projection(fmt, io, M, K, N):
    x = _x(M, K, io, seed=M + K)
    w, ws = _weights(fmt, N, K, seed=N)
    ratio, ulp = _check(fmt, x, w, ws, N)
    print("%s io=%s M=%d K=%d N=%d: err/bound %.3f, bf16 out %d ulp"
          % (fmt, io, M, K, N, ratio, ulp))
    assert ratio <= 1.0 and ulp <= 1


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("M", [1500, 4097])
def test_fp8_projection_one_step(io, M):
    """FP8 with K = 128, a single K step: the tile kernel (1500 tokens) and
    the 256 x 256 GEMM (4097 tokens, every load after the first re-reading
    that step, the pipelined halves at their edge)."""
    K, N = 128, 36
    x = _x(M, K, io, seed=17)
    w, ws = _weights("fp8", N, K, seed=N)
    ratio, ulp = _check("fp8", x, w, ws, N)
    print("fp8 io=%s M=%d K=%d N=%d: err/bound %.3f, bf16 out %d ulp" % (io, M, K, N, ratio, ulp))
    assert ratio <= 1.0 and ulp <= 1


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_lowp_layer_shapes(fmt):
    """4096 -> 2048 at the 256-token decode batch (all rows) and the
    32768-token prefill (first, last and 254 random rows); also the error of
    the quantized projection against the unquantized one, for the record."""
    K, N = 4096, 2048
    w, ws = _weights(fmt, N, K, seed=11)
    for M, ns in ((256, 256), (32768, 254)):
        x = _x(M, K, "bf16", seed=M, spread=False)
        rng = np.random.default_rng(M)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, ns, replace=False)]))
        ratio, ulp = _check(fmt, x, w, ws, N, rows=rows)
        print("%s M=%d: err/bound %.3f over %d rows, bf16 out %d ulp"
              % (fmt, M, ratio, rows.size, ulp))
        assert ratio <= 1.0 and ulp <= 1
