"""Pins of the Q4_K projection oracle (oracle/q4k.py) against facts that do
not come from the oracle itself: the block and payload sizes the page prints,
the bit structure of the packing (every stored bit reaches exactly one field
or value), closed forms for constant quants, a packer written independently
from the packing side, and the projection's orientation and definition by
brute force."""
import numpy as np

from oracle import q4k as Q

RNG = np.random.default_rng(4321)


def _block(d=1.0, dmin=0.5, s12=None, qs=None):
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
    blk[4:16] = RNG.integers(0, 256, 12) if s12 is None else s12
    blk[16:] = RNG.integers(0, 256, 128) if qs is None else qs
    return blk


def _payload(nblocks):
    """Random blocks with finite fp16 d and dmin (random bytes there could
    be NaN or infinity)."""
    wq = RNG.integers(0, 256, (nblocks, 144), dtype=np.uint8)
    dd = RNG.uniform(-1, 1, (nblocks, 2)).astype(np.float16)
    wq[:, 0:4] = dd.view(np.uint8).reshape(nblocks, 4)
    return wq.reshape(-1)


def _pack(d, dmin, sc, mn, q):
    """Independent packer, written from the packing side: six-bit fields
    0-3 fill the low bits of bytes 0-3 (scales) and 4-7 (mins); fields 4-7
    put their low four bits in bytes 8-11 (scale low nibble, min high nibble)
    and their top two bits in the spare top bits of bytes 0-3 (scales) and
    4-7 (mins).  Quant run p (32 bytes) carries sub-block 2p in its low
    nibbles and 2p+1 in its high nibbles."""
    s = [0] * 12
    for j in range(4):
        s[j] |= sc[j]
        s[4 + j] |= mn[j]
        s[j] |= (sc[4 + j] >> 4) << 6
        s[4 + j] |= (mn[4 + j] >> 4) << 6
        s[8 + j] = (sc[4 + j] & 15) | ((mn[4 + j] & 15) << 4)
    qs = np.zeros(128, np.uint8)
    for p in range(4):
        lo = q[64 * p:64 * p + 32]
        hi = q[64 * p + 32:64 * p + 64]
        qs[32 * p:32 * p + 32] = lo | (hi << 4)
    return _block(d, dmin, np.array(s, np.uint8), qs)


def test_sizes_printed_on_the_page():
    """256 values in 144 bytes (2 + 2 + 12 + 128); a 4096-value row is 16
    blocks = 2304 bytes; the 4096 x 2048 weight is 4.5 MiB."""
    assert Q.BLOCK_BYTES == 2 + 2 + 12 + 128 == 144 and Q.BLOCK_VALUES == 256
    assert (4096 // Q.BLOCK_VALUES) * Q.BLOCK_BYTES == 2304
    assert 2048 * 2304 == int(4.5 * 2**20)
    wq = _payload(3 * 16)
    W = Q.decode_matrix(wq, 3, 4096)
    assert W.shape == (3, 4096)
    for r in range(3):       # row r is its own 2304 bytes
        assert np.array_equal(W[r, :256], Q.decode_block(wq[r * 2304:r * 2304 + 144]))
    try:
        Q.decode_matrix(wq[:-1], 3, 4096)
        assert False, "a short payload must be rejected"
    except (ValueError, AssertionError):
        pass


def test_scale_bytes_are_a_bit_permutation():
    """Each of the 96 bits of the 12 scale bytes changes exactly one of the
    16 six-bit fields by exactly one power of two, and no two bits reach the
    same (field, bit): the packing loses and duplicates nothing."""
    base = RNG.integers(0, 256, 12).astype(np.uint8)
    sc0, mn0 = Q.scales_mins(base)
    hit = set()
    for byte in range(12):
        for bit in range(8):
            s = base.copy()
            s[byte] ^= (1 << bit)
            sc, mn = Q.scales_mins(s)
            diffs = [(f, abs(a - b)) for f, (a, b) in
                     enumerate(zip(sc + mn, sc0 + mn0)) if a != b]
            assert len(diffs) == 1
            f, delta = diffs[0]
            b = int(np.log2(delta))
            assert delta == 1 << b and b < 6
            hit.add((f, b))
    assert len(hit) == 96
    assert all(0 <= v < 64 for v in sc0 + mn0)


def test_quant_bits_reach_one_value_each():
    """Each of the 1024 quant bits changes exactly one of the 256 values, by
    d * scale * 2^b of that value's sub-block; values of sub-block j sit at
    positions 32j .. 32j+31."""
    s12 = RNG.integers(0, 256, 12).astype(np.uint8)
    sc, _ = Q.scales_mins(s12)
    sc = [max(v, 1) for v in sc]
    # force every scale nonzero so that every flip is visible
    s12[0:4] = (s12[0:4] & 0xC0) | np.array(sc[:4], np.uint8)
    s12[8:12] = (s12[8:12] & 0xF0) | (np.array(sc[4:], np.uint8) & 15)
    s12[0:4] |= ((np.array(sc[4:], np.uint8) >> 4) << 6).astype(np.uint8)
    sc, _ = Q.scales_mins(s12)
    assert min(sc) >= 1
    blk = _block(2.0, 0.25, s12)
    v0 = Q.decode_block(blk)
    seen = set()
    for byte in range(128):
        for bit in range(8):
            b2 = blk.copy()
            b2[16 + byte] ^= (1 << bit)
            dv = Q.decode_block(b2) - v0
            idx = np.nonzero(dv)[0]
            assert idx.size == 1
            i = int(idx[0])
            assert abs(dv[i]) == 2.0 * sc[i // 32] * (1 << (bit % 4))
            seen.add((i, bit % 4))
    assert len(seen) == 1024


def test_closed_forms_constant_quants():
    s12 = RNG.integers(0, 256, 12).astype(np.uint8)
    sc, mn = Q.scales_mins(s12)
    v = Q.decode_block(_block(1.5, 0.75, s12, np.zeros(128, np.uint8)))
    assert np.array_equal(v, np.repeat([-0.75 * m for m in mn], 32))
    v = Q.decode_block(_block(1.5, 0.75, s12, np.full(128, 0xFF, np.uint8)))
    assert np.array_equal(v, np.repeat([1.5 * 15 * s - 0.75 * m
                                        for s, m in zip(sc, mn)], 32))
    assert not np.any(Q.decode_block(_block(0.0, 0.0)))
    # a negative super-block scale flips the quant term only
    qs = RNG.integers(0, 256, 128).astype(np.uint8)
    a = Q.decode_block(_block(1.0, 0.5, s12, qs))
    b = Q.decode_block(_block(-1.0, 0.5, s12, qs))
    c = Q.decode_block(_block(0.0, 0.5, s12, qs))
    assert np.allclose(a + b, 2 * c, rtol=0, atol=0)


def test_independent_packer_round_trip():
    for trial in range(20):
        d = float(np.float16(RNG.uniform(-2, 2)))
        dmin = float(np.float16(RNG.uniform(0, 1)))
        sc = [int(v) for v in RNG.integers(0, 64, 8)]
        mn = [int(v) for v in RNG.integers(0, 64, 8)]
        if trial == 0:
            sc, mn = [63] * 8, [63] * 8
        q = RNG.integers(0, 16, 256).astype(np.uint8)
        v = Q.decode_block(_pack(d, dmin, sc, mn, q))
        want = np.array([d * sc[i // 32] * int(q[i]) - dmin * mn[i // 32]
                         for i in range(256)])
        assert np.array_equal(v, want)


def test_projection_orientation_one_hot():
    """x = e_k picks value k of every weight row: y[n] = W[n, k]; the weight
    is stored [out_features rows, in_features values]."""
    N, K = 3, 512
    wq = _payload(N * (K // 256))
    for k in (0, 31, 32, 255, 256, 300, 511):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        y = Q.project(x, wq, N)
        assert y.shape == (1, N)
        for n in range(N):
            blk = wq[(n * 2 + k // 256) * 144:(n * 2 + k // 256 + 1) * 144]
            assert y[0, n] == Q.decode_block(blk)[k % 256]


def test_projection_brute_force():
    M, N, K = 2, 3, 256
    wq = _payload(N)
    x = RNG.standard_normal((M, K))
    y = Q.project(x, wq, N)
    for m in range(M):
        for n in range(N):
            w = Q.decode_block(wq[n * 144:(n + 1) * 144])
            acc = 0.0
            for k in range(K):
                acc += x[m, k] * w[k]
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_dense_projection_matches_dequantized():
    """The dense form with the dequantized matrix as its weight equals the
    Q4_K form, and a one-hot input picks a weight column."""
    N, K = 5, 256
    wq = _payload(N)
    W = np.stack([Q.decode_block(wq[n * 144:(n + 1) * 144]) for n in range(N)])
    x = RNG.standard_normal((3, K))
    assert np.array_equal(Q.project_dense(x, W), Q.project(x, wq, N))
    e = np.zeros((1, K))
    e[0, 7] = 1.0
    assert np.array_equal(Q.project_dense(e, W)[0], W[:, 7])
