"""Parity metrics shared by the GPU tests.

Reading of "max relative error" used throughout: for every (sequence, value
head) slice, err = max |x - y| / max |y| (infinity-norm-wise), with y the
fp64 oracle.  It is applied to the fp32 final state directly and to outputs
produced in fp32 (out_dtype = f32, the same kernels with a wider final
store).  A bf16 output must then equal the round-to-nearest-even bf16 of the
fp32 output to within one bf16 ulp: a bf16 store alone carries up to 2^-9
relative rounding, more than the 2e-3 budget, so bf16 values are not held to
it directly.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_BF16_INPUTS = 2e-3   # bf16 inputs, fp32 state
TOL_F32_INPUTS = 1e-5    # fp32 inputs


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_inf(x, y) -> float:
    x, y = to_np(x), to_np(y)
    if y.size == 0:
        return 0.0
    den = float(np.max(np.abs(y)))
    num = float(np.max(np.abs(x - y)))
    return num / den if den > 0 else num


def per_head_rel(out, ref, cu, h_v, d_v) -> float:
    """Max over (sequence, value head) of the slice error of [T, h_v*d_v] or
    [T, h_v, d_v] outputs."""
    out = to_np(out).reshape(-1, h_v, d_v)
    ref = to_np(ref).reshape(-1, h_v, d_v)
    worst = 0.0
    for n in range(len(cu) - 1):
        for h in range(h_v):
            worst = max(worst, rel_inf(out[cu[n]:cu[n + 1], h],
                                       ref[cu[n]:cu[n + 1], h]))
    return worst


def rowwise_rel(out, ref, width) -> float:
    """Max over consecutive groups of `width` values (one head of one token,
    or one state row block) of max|x - y| / max|y| -- vectorised."""
    out = to_np(out).reshape(-1, width)
    ref = to_np(ref).reshape(-1, width)
    num = np.max(np.abs(out - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


def per_state_rel(st, ref) -> float:
    st, ref = to_np(st), to_np(ref)
    st = st.reshape(-1, st.shape[-2], st.shape[-1])
    ref = ref.reshape(-1, ref.shape[-2], ref.shape[-1])
    return max((rel_inf(st[i], ref[i]) for i in range(st.shape[0])),
               default=0.0)


def bf16_ulp_diff(bf16_out: torch.Tensor, f32_out: torch.Tensor) -> int:
    """Largest distance in bf16 ulps between a bf16 tensor and the RNE bf16
    of an fp32 tensor (0 means bit-identical)."""
    a = bf16_out.detach().contiguous().view(torch.int16).cpu().numpy()
    b = f32_out.detach().to(torch.bfloat16).contiguous().view(
        torch.int16).cpu().numpy()

    def ordered(v):
        v = v.astype(np.int32)
        return np.where(v < 0, -(v & 0x7FFF), v)
    if a.size == 0:
        return 0
    return int(np.max(np.abs(ordered(a) - ordered(b))))
