"""fp64 CPU oracle of the low-precision projections (W8A8 FP8, W4A4 MXFP4).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the benchmark's check
code; never by the library or its binding.

"Why Gated DeltaNet Survives 4-Bit Quantization", Abstract: every linear
layer of the hybrid model, the GDN block's included, runs with 4-bit weights
and activations under block scaling, and the recurrence itself stays in high
precision.  The pages use NVFP4 on other hardware; the matrix cores of this
GPU take the OCP formats natively, so the projections here are:

  * FP8 W8A8: E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; no infinities, S.1111.111 is NaN, max 448, subnormals m/8 * 2^-6).
    Activations: one power-of-two scale per token, the smallest 2^e with
    max|x| / 2^e <= 448 (but e >= -126); codes are x / 2^e rounded to
    nearest even.  Weights:
    E4M3 codes with one fp32 scale per output row.
  * MXFP4 W4A4 (OCP Microscaling): blocks of 32 consecutive values along K
    share an E8M0 scale 2^(s - 127); elements are E2M1 (1 sign, 2 exponent
    bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The block
    scale exponent is floor(log2(max|v|)) - 2 (2 being the largest E2M1
    exponent), elements are v / scale rounded to nearest even and saturated
    at 6; an all-zero block takes scale 2^0.

Every division by a scale is by a power of two, so it is exact and both
implementations take their rounding decisions on the same values.  The
projection is y = dequant(x) dequant(W)^T in fp64.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


# ------------------------------------------------------------------ E4M3 --
def e4m3_decode(code: int) -> float:
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _round_half_even(x: float) -> int:
    f = math.floor(x)
    r = x - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        return f + 1
    return f


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 code (ties to an even mantissa); |v| must be <= 448."""
    sign = 0x80 if (v < 0 or (v == 0 and math.copysign(1.0, v) < 0)) else 0
    a = abs(v)
    assert a <= E4M3_MAX, a
    if a < 2.0 ** -6:                      # subnormal range, step 2^-9
        m = _round_half_even(a / 2.0 ** -9)
        return sign | m if m < 8 else sign | (1 << 3)
    e = math.floor(math.log2(a))
    if 2.0 ** (e + 1) <= a:                # guard log2 rounding
        e += 1
    if 2.0 ** e > a:
        e -= 1
    m = _round_half_even((a / 2.0 ** e - 1.0) * 8.0)
    if m == 8:
        e, m = e + 1, 0
    return sign | ((e + 7) << 3) | m


def fp8_row_scale_exp(amax: float) -> int:
    """Smallest e with amax / 2^e <= 448, but at least -126 so that 2^e is a
    normal fp32 number (0 for an all-zero row)."""
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax / 2.0 ** e > E4M3_MAX:
        e += 1
    while e > -200 and amax / 2.0 ** (e - 1) <= E4M3_MAX:
        e -= 1
    return max(e, -126)


def quantize_rows_fp8(x):
    """x [M, K] -> (codes uint8 [M, K], scale exponents int [M])."""
    x = np.asarray(x, np.float64)
    M, K = x.shape
    codes = np.zeros((M, K), np.uint8)
    exps = np.zeros(M, np.int64)
    for m in range(M):
        e = fp8_row_scale_exp(float(np.max(np.abs(x[m]))) if K else 0.0)
        exps[m] = e
        for k in range(K):
            codes[m, k] = e4m3_encode(float(x[m, k]) / 2.0 ** e)
    return codes, exps


def dequant_fp8(codes, row_scale):
    """codes [R, K] with a per-row multiplier [R] -> fp64 [R, K]."""
    table = np.array([e4m3_decode(c) for c in range(256)])
    return table[np.asarray(codes, np.int64)] * np.asarray(row_scale,
                                                          np.float64)[:, None]


# ------------------------------------------------------------------ E2M1 --
def e2m1_decode(code: int) -> float:
    code = int(code) & 15
    v = E2M1_VALUES[code & 7]
    return -v if code & 8 else v


def e2m1_encode(v: float) -> int:
    """Nearest E2M1 code, ties to an even mantissa, saturating at 6."""
    sign = 8 if v < 0 else 0
    a = abs(v)
    if a >= 6.0:
        return sign | 7
    if a < 1.0:                            # 0 or 0.5 (subnormal), step 0.5
        n = _round_half_even(a / 0.5)      # 0, 1 or 2
        return sign | n                    # code 2 is 1.0
    e = math.floor(math.log2(a))           # 0, 1 or 2
    m = _round_half_even((a / 2.0 ** e - 1.0) * 2.0)
    if m == 2:
        e, m = e + 1, 0
    if e > 2:
        return sign | 7
    return sign | ((e + 1) << 1) | m


def mx_block_scale_code(amax: float) -> int:
    """E8M0 code of a block's scale: 127 + floor(log2(amax)) - 2."""
    if amax == 0.0:
        return 127
    e = math.floor(math.log2(amax))
    if 2.0 ** (e + 1) <= amax:
        e += 1
    if 2.0 ** e > amax:
        e -= 1
    return int(min(254, max(0, 127 + e - 2)))


def quantize_rows_mxfp4(x):
    """x [M, K] (K % 32 == 0) -> (codes uint8 [M, K] one per value,
    scale codes uint8 [M, K / 32])."""
    x = np.asarray(x, np.float64)
    M, K = x.shape
    codes = np.zeros((M, K), np.uint8)
    scales = np.zeros((M, K // 32), np.uint8)
    for m in range(M):
        for b in range(K // 32):
            blk = x[m, 32 * b:32 * b + 32]
            s = mx_block_scale_code(float(np.max(np.abs(blk))))
            scales[m, b] = s
            for i in range(32):
                codes[m, 32 * b + i] = e2m1_encode(float(blk[i]) / 2.0 ** (s - 127))
    return codes, scales


def pack_fp4(codes):
    """One code per value [R, K] -> two per byte [R, K / 2], even k in the
    low nibble."""
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed):
    packed = np.asarray(packed, np.uint8)
    out = np.zeros((packed.shape[0], packed.shape[1] * 2), np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


def dequant_mxfp4(codes, scales):
    """codes [R, K] one per value, scales [R, K / 32] -> fp64 [R, K]."""
    table = np.array([e2m1_decode(c) for c in range(16)])
    vals = table[np.asarray(codes, np.int64)]
    sc = 2.0 ** (np.asarray(scales, np.float64) - 127.0)
    return vals * np.repeat(sc, 32, axis=1)


# ----------------------------------------------------------- projections --
def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, np.float64)


def project_fp8(x, w_codes, w_scale):
    """W8A8: activations quantized per token, weight codes with per-row
    scales.  Returns (y [M, N], x codes, x scale exponents)."""
    xc, xe = quantize_rows_fp8(_f64(x))
    X = dequant_fp8(xc, 2.0 ** xe.astype(np.float64))
    W = dequant_fp8(_u8(w_codes), _f64(w_scale))
    return X @ W.T, xc, xe


def project_mxfp4(x, w_packed, w_scales):
    """W4A4 MXFP4.  Returns (y [M, N], x codes packed, x scale codes)."""
    xc, xs = quantize_rows_mxfp4(_f64(x))
    X = dequant_mxfp4(xc, xs)
    W = dequant_mxfp4(unpack_fp4(_u8(w_packed)), _u8(w_scales))
    return X @ W.T, pack_fp4(xc), xs


def _u8(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a, np.uint8)


def abs_product(x_deq, w_deq):
    """sum_k |x_k w_k| per output: the scale of an fp32 dot product's
    rounding error bound."""
    return np.abs(x_deq) @ np.abs(w_deq).T
