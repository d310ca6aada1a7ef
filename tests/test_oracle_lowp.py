"""Pins of the low-precision projection oracle (oracle/lowp.py) against facts
that do not come from it: torch's own float8_e4m3fn decoding and rounding,
the E2M1 value table of the OCP Microscaling format and a brute-force
nearest-value search, the defining inequalities of the scale choices, and
brute-force projections."""
import math

import numpy as np
import torch

from oracle import lowp as L

RNG = np.random.default_rng(777)


def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([L.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert max(ours[~nan]) == 448.0 and min(abs(ours[1:127])) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rounding():
    """Random values, every midpoint between neighbouring codes (ties go to
    the even mantissa) and points just beside them, over the whole range."""
    finite = sorted({L.e4m3_decode(c) for c in range(256)} - {float("nan")})
    finite = [v for v in finite if not math.isnan(v)]
    mids = [(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])]
    vals = np.concatenate([RNG.uniform(-448, 448, 3000),
                           RNG.standard_normal(3000) * 2.0 ** RNG.integers(-12, 8, 3000),
                           mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                           finite]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([L.e4m3_encode(float(v)) for v in vals], np.uint8)
    # torch keeps the sign of a value that rounds to zero; so do we
    assert np.array_equal(ours, ref)


def test_fp8_row_scale_is_the_tightest_power_of_two():
    for amax in np.concatenate([RNG.uniform(0, 1, 200) * 10.0 ** RNG.integers(-8, 8, 200),
                                [448.0, 448.0 * 2 ** 5, 1.0, 2.0 ** -20, 449.0]]):
        e = L.fp8_row_scale_exp(float(amax))
        assert amax / 2.0 ** e <= 448.0 < amax / 2.0 ** (e - 1)
    assert L.fp8_row_scale_exp(0.0) == 0
    assert L.fp8_row_scale_exp(1e-40) == -126       # floor: 2^e stays normal


def test_e2m1_table_and_bruteforce_rounding():
    """Codes 0..7 are the OCP E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
    encoding picks the nearest magnitude, a tie going to the code with an
    even mantissa bit, and saturates at 6."""
    assert [L.e2m1_decode(c) for c in range(8)] == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert [L.e2m1_decode(c) for c in range(8, 16)] == [-0.0, -.5, -1, -1.5, -2, -3, -4, -6]

    def brute(v):
        best = None
        for c in range(16):
            d = abs(L.e2m1_decode(c) - v)
            key = (d, c & 1)                     # prefer the even mantissa
            if (v < 0) != bool(c & 8) and v != 0:
                continue
            if best is None or key < best[0]:
                best = (key, c)
        return best[1]
    grid = np.arange(-8.0, 8.0 + 1e-9, 0.125)
    vals = np.concatenate([grid, RNG.uniform(-7, 7, 2000)])
    for v in vals:
        c = L.e2m1_encode(float(v))
        if abs(v) >= 6:
            assert c & 7 == 7
        elif v != 0:
            assert c == brute(float(v)), (v, c, brute(float(v)))
    assert L.e2m1_encode(2.5) == 4 and L.e2m1_encode(5.0) == 6
    assert L.e2m1_encode(0.25) == 0 and L.e2m1_encode(0.75) == 2


def test_mx_block_scale_puts_the_block_max_in_4_to_8():
    for amax in RNG.uniform(0, 1, 300) * 10.0 ** RNG.integers(-20, 20, 300):
        s = L.mx_block_scale_code(float(amax))
        r = amax / 2.0 ** (s - 127)
        assert 4.0 <= r < 8.0
    assert L.mx_block_scale_code(0.0) == 127


def test_fp4_packing_low_nibble_first():
    codes = RNG.integers(0, 16, (3, 64)).astype(np.uint8)
    packed = L.pack_fp4(codes)
    assert packed.shape == (3, 32)
    assert np.array_equal(packed[:, 5] & 15, codes[:, 10])
    assert np.array_equal(packed[:, 5] >> 4, codes[:, 11])
    assert np.array_equal(L.unpack_fp4(packed), codes)


def test_quantization_error_bounds():
    x = RNG.standard_normal((4, 256))
    xc, xe = L.quantize_rows_fp8(x)
    X = L.dequant_fp8(xc, 2.0 ** xe.astype(float))
    rel = np.abs(X - x)
    # 3 mantissa bits: within 2^-4 relative for normals; subnormal step 2^-9 * 2^e
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** (xe[:, None] - 10))
    assert np.all(rel <= bound)
    qc, qs = L.quantize_rows_mxfp4(x)
    Q = L.dequant_mxfp4(qc, qs)
    step = np.repeat(2.0 ** (qs.astype(float) - 127), 32, axis=1)
    assert np.all(np.abs(Q - x) <= 2.0 * step)      # saturation at 6 of 8
    inside = np.abs(x) <= 6 * step
    assert np.all((np.abs(Q - x) <= step)[inside])


def test_projections_brute_force_and_orientation():
    M, N, K = 2, 3, 64
    x = RNG.standard_normal((M, K))
    wc = RNG.integers(0, 256, (N, K)).astype(np.uint8)
    wc[(wc & 0x7F) == 0x7F] = 0x38
    ws = RNG.uniform(0.01, 0.1, N)
    y, xc, xe = L.project_fp8(x, wc, ws)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += (L.e4m3_decode(xc[m, k]) * 2.0 ** xe[m]) * (L.e4m3_decode(wc[n, k]) * ws[n])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    wq = RNG.integers(0, 16, (N, K)).astype(np.uint8)
    wsc = RNG.integers(120, 130, (N, K // 32)).astype(np.uint8)
    y4, xp, xs = L.project_mxfp4(x, L.pack_fp4(wq), wsc)
    xq = L.unpack_fp4(xp)
    for m in range(M):
        for n in range(N):
            acc = sum(L.e2m1_decode(xq[m, k]) * 2.0 ** (int(xs[m, k // 32]) - 127)
                      * L.e2m1_decode(wq[n, k]) * 2.0 ** (int(wsc[n, k // 32]) - 127)
                      for k in range(K))
            assert abs(y4[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    # one-hot activation row picks weight column k of every output row
    e = np.zeros((1, K))
    e[0, 40] = 1.0
    y1, _, _ = L.project_fp8(e, wc, ws)
    assert np.allclose(y1[0], [L.e4m3_decode(wc[n, 40]) * ws[n] for n in range(N)], rtol=0, atol=0)
