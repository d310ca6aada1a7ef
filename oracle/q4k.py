"""fp64 CPU oracle of the Q4_K output projection that follows the tail.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the benchmark's check
code; never by the library or its binding.

"Red Lite dev15d -- DeltaNet gated tail + Q4_K output projection":
  * Scope / Pinned graph semantics step 6: the flattened 4096-value tail
    output is multiplied by ssm_out (4096 -> 2048);
  * Q4_K implementation: blocks of 256 values in 144 bytes -- fp16 d, fp16
    dmin, 12 bytes packing eight 6-bit scales and eight 6-bit mins, 128
    bytes of 4-bit quants; a 4096-value row is 16 blocks (2304 bytes).

The page pins the canonical GGUF Q4_K layout without spelling out its bit
order; this oracle reads it as follows (the published format):
  * sub-block j (32 values) has scale sc_j and min m_j, 6 bits each.  For
    j < 4: sc_j = s[j] & 63, m_j = s[j+4] & 63.  For j >= 4 the low four bits
    sit in s[j+4] (sc in the low nibble, m in the high nibble) and the top two
    bits in the top bits of s[j-4] (sc) and s[j] (m);
  * the 128 quant bytes come in four runs of 32: run p holds sub-block 2p in
    its low nibbles and sub-block 2p+1 in its high nibbles, value l of the
    sub-block being byte l of the run;
  * value = d * sc_j * q - dmin * m_j.
"""
from __future__ import annotations

import numpy as np

BLOCK_VALUES = 256
BLOCK_BYTES = 144


def _u8(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.uint8)


def scales_mins(s12):
    """The eight (scale, min) pairs packed in 12 bytes."""
    s = [int(b) for b in s12]
    sc, mn = [0] * 8, [0] * 8
    for j in range(8):
        if j < 4:
            sc[j] = s[j] & 63
            mn[j] = s[j + 4] & 63
        else:
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4)
            mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)
    return sc, mn


def decode_block(blk):
    """256 fp64 values of one 144-byte block."""
    blk = _u8(blk).reshape(-1)
    assert blk.size == BLOCK_BYTES
    d = float(blk[0:2].view(np.float16)[0])
    dmin = float(blk[2:4].view(np.float16)[0])
    sc, mn = scales_mins(blk[4:16])
    qs = blk[16:144]
    out = np.empty(BLOCK_VALUES)
    for p in range(4):
        run = qs[32 * p:32 * p + 32].astype(np.int64)
        for half, j in ((0, 2 * p), (1, 2 * p + 1)):
            q = (run & 15) if half == 0 else (run >> 4)
            out[64 * p + 32 * half:64 * p + 32 * half + 32] = (
                d * sc[j] * q - dmin * mn[j])
    return out


def decode_matrix(wq, rows, cols):
    """Dequantized [rows, cols] fp64 matrix from Q4_K bytes laid out row
    after row, each row cols / 256 blocks."""
    wq = _u8(wq).reshape(rows, cols // BLOCK_VALUES, BLOCK_BYTES)
    out = np.empty((rows, cols))
    for r in range(rows):
        for b in range(cols // BLOCK_VALUES):
            out[r, b * 256:(b + 1) * 256] = decode_block(wq[r, b])
    return out


def project(x, wq, out_features):
    """y = x W^T with W the dequantized [out_features, in_features] matrix;
    x: [T, in_features] (any float dtype, taken exactly in fp64)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    x = np.asarray(x, dtype=np.float64)
    W = decode_matrix(wq, out_features, x.shape[1])
    return x @ W.T


def project_dense(x, w):
    """The same projection with a dense [out_features, in_features] weight
    (e.g. bf16, taken exactly in fp64): y = x W^T."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    if hasattr(w, "detach"):
        w = w.detach().cpu().double().numpy()
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
