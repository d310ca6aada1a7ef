"""Seeded synthetic inputs for the gated delta-rule layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no gates, no recurrence, no norm), so both the HIP path and
the CPU oracle can be fed from it without sharing any of the method.

Distributions follow the layer's workloads:
  * q, k ~ N(0, 1), L2-normalised per (token, key head) in fp32 and then cast
    to the io dtype (round to nearest even for bf16);
  * v, z ~ N(0, 1) cast to the io dtype;
  * g, beta ~ N(0, 1) per (token, value head), fp32 gate pre-activations;
  * "tiny" gate parameters: A_log ~ U(0, ln 16), dt_bias ~ U(-2, 0) per head;
  * "spread" gate parameters: dt_bias ~ U(-2, 0) and A_log log-spaced over the
    heads so that the decay at zero pre-activation, exp(-exp(A_log) * ln 2),
    runs from 0.999 (first head) to 0.001 (last head) -- the fixed spectrum
    of forget-gate time scales, ~0.001 to 1.0, that the white-box walkthrough
    of a quantized hybrid GDN model reports in its results on gates;
  * norm weight w ~ U(0.5, 1.5) [d_v] fp32;
  * initial state ~ N(0, std^2) fp32 when requested.
Draw order is fixed: q, k, v, z, g, beta, A_log/dt_bias, w, S0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

F32 = "f32"
BF16 = "bf16"


def torch_dtype(io: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16}[io]


@dataclass
class Workload:
    """Shape and recipe of one synthetic workload."""
    name: str
    lens: List[int]              # tokens per sequence (decode: [1] * N)
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    io: str = BF16
    chunk: int = 64
    gates: str = "spread"        # "tiny" or "spread"
    tail: bool = False
    s0_std: Optional[float] = None
    eps: float = 1e-6
    seed: int = 0
    decode: bool = False
    notes: str = ""

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lens))

    @property
    def n_seqs(self) -> int:
        return len(self.lens)

    def cu_seqlens(self) -> List[int]:
        cu = [0]
        for n in self.lens:
            cu.append(cu[-1] + int(n))
        return cu


# The five workloads of the layer at the sizes the library is measured on.
WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", [64], 2, 2, 16, 16, io=F32, chunk=16, gates="tiny",
        seed=0, notes="B=1, T=64, H=2, d=16, fp32, chunk 16, zero state"),
    "prefill_t4096_h8": Workload(
        "prefill_t4096_h8", [4096], 8, 8, 128, 128, io=BF16, chunk=64,
        seed=1, notes="B=1, T=4096, H=8, d=128, bf16, chunk 64, zero state"),
    "prefill_t32768_hv32_tail": Workload(
        "prefill_t32768_hv32_tail", [32768], 16, 32, 128, 128, io=BF16,
        chunk=64, tail=True, seed=2,
        notes="B=1, T=32768, 32 value / 16 key heads, d=128, bf16, fused "
              "gated-RMSNorm tail, output [T, 4096]"),
    "decode_n256_hv32": Workload(
        "decode_n256_hv32", [1] * 256, 16, 32, 128, 128, io=BF16, tail=True,
        s0_std=0.05, seed=3, decode=True,
        notes="256 sequences x 1 token, 32 value / 16 key heads, d=128, "
              "fp32 state [256,32,128,128] in place, fused tail"),
    "varlen_8seq_hv32": Workload(
        "varlen_8seq_hv32",
        [1024, 2048, 4096, 8192, 16384, 32768, 65536, 1000], 16, 32, 128, 128,
        io=BF16, chunk=64, tail=True, s0_std=0.05, seed=4,
        notes="8 packed sequences (131048 tokens), 32 value / 16 key heads, "
              "d=128, bf16, carried fp32 state, fused tail"),
}
WORKLOAD_ORDER = ["tiny_fp32", "prefill_t4096_h8", "prefill_t32768_hv32_tail",
                  "decode_n256_hv32", "varlen_8seq_hv32"]


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    z: Optional[torch.Tensor] = None
    w: Optional[torch.Tensor] = None
    s0: Optional[torch.Tensor] = None
    cu_seqlens: Optional[torch.Tensor] = None
    cu_list: List[int] = field(default_factory=list)
    eps: float = 1e-6


def _l2n(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def gate_params(h_v: int, recipe: str, gen: torch.Generator, device):
    """Per-head A_log and dt_bias (fp32)."""
    if recipe == "tiny":
        A_log = torch.rand(h_v, generator=gen, device=device) * math.log(16.0)
        dt_bias = torch.rand(h_v, generator=gen, device=device) * 2.0 - 2.0
        return A_log, dt_bias
    if recipe == "spread":
        dt_bias = torch.rand(h_v, generator=gen, device=device) * 2.0 - 2.0
        lo, hi = math.log(1e-3), math.log(-math.log(1e-3))
        frac = torch.arange(h_v, dtype=torch.float64) / max(h_v - 1, 1)
        lam = torch.exp(lo + (hi - lo) * frac)
        A_log = torch.log(lam / math.log(2.0)).to(torch.float32).to(device)
        return A_log, dt_bias
    raise ValueError("unknown gate recipe %r" % recipe)


def make_inputs(wl: Workload, device="cpu", seed: Optional[int] = None,
                lens: Optional[List[int]] = None) -> Inputs:
    """Draw the inputs of workload ``wl`` (optionally with other lengths)."""
    lens = list(wl.lens if lens is None else lens)
    T = int(sum(lens))
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed if seed is None else seed)
    dt = torch_dtype(wl.io)
    f32 = torch.float32
    q = _l2n(torch.randn(T, wl.h_k, wl.d_k, generator=gen, device=device,
                         dtype=f32)).to(dt)
    k = _l2n(torch.randn(T, wl.h_k, wl.d_k, generator=gen, device=device,
                         dtype=f32)).to(dt)
    v = torch.randn(T, wl.h_v, wl.d_v, generator=gen, device=device,
                    dtype=f32).to(dt)
    z = None
    if wl.tail:
        z = torch.randn(T, wl.h_v, wl.d_v, generator=gen, device=device,
                        dtype=f32).to(dt)
    g = torch.randn(T, wl.h_v, generator=gen, device=device, dtype=f32)
    beta = torch.randn(T, wl.h_v, generator=gen, device=device, dtype=f32)
    A_log, dt_bias = gate_params(wl.h_v, wl.gates, gen, device)
    w = None
    if wl.tail:
        w = torch.rand(wl.d_v, generator=gen, device=device, dtype=f32) + 0.5
    s0 = None
    if wl.s0_std is not None:
        s0 = torch.randn(len(lens), wl.h_v, wl.d_v, wl.d_k, generator=gen,
                         device=device, dtype=f32) * wl.s0_std
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    cu_t = torch.tensor(cu, dtype=torch.int32, device=device)
    return Inputs(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias,
                  z=z, w=w, s0=s0, cu_seqlens=cu_t, cu_list=cu, eps=wl.eps)


def random_case(*, T_list, h_k, h_v, d_k, d_v, io=BF16, seed=0, gates="spread",
                tail=False, s0_std=None, device="cpu") -> Inputs:
    """Inputs for an ad-hoc shape (tests)."""
    wl = Workload("case", list(T_list), h_k, h_v, d_k, d_v, io=io, gates=gates,
                  tail=tail, s0_std=s0_std, seed=seed)
    return make_inputs(wl, device=device)


def q4k_weight(out_features: int, in_features: int, seed: int = 0,
               d_scale: float = 1e-4, subnormal_rows: int = 0,
               device="cpu") -> torch.Tensor:
    """Random packed Q4_K weight bytes [out_features, in_features / 256 * 144]
    (uint8), blocks back to back along each row.  Per block: fp16 d ~
    U(0.5, 1.5) * d_scale and dmin ~ U(0.5, 1.5) * 2 * d_scale (so that
    values are of order 1e-2, like a projection weight), the 12 scale/min
    bytes and the 128 quant bytes uniform random bytes.  The first
    `subnormal_rows` rows draw d and dmin below the fp16 normal range
    (subnormal halves)."""
    import numpy as np
    assert in_features % 256 == 0
    nb = out_features * (in_features // 256)
    rng = np.random.default_rng(seed)
    raw = rng.integers(0, 256, size=(nb, 144), dtype=np.uint8)
    d = rng.uniform(0.5, 1.5, nb) * d_scale
    dmin = rng.uniform(0.5, 1.5, nb) * 2 * d_scale
    ns = subnormal_rows * (in_features // 256)
    d[:ns] = rng.uniform(1e-7, 6e-5, ns)
    dmin[:ns] = rng.uniform(1e-7, 6e-5, ns)
    raw[:, 0:2] = d.astype(np.float16).view(np.uint8).reshape(nb, 2)
    raw[:, 2:4] = dmin.astype(np.float16).view(np.uint8).reshape(nb, 2)
    t = torch.from_numpy(raw.reshape(out_features, -1).copy())
    return t.to(device)


def dense_weight(out_features: int, in_features: int, seed: int = 0,
                 std: float = 0.02, device="cpu") -> torch.Tensor:
    """bf16 [out_features, in_features] ~ N(0, std^2)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    w = torch.randn(out_features, in_features, generator=gen) * std
    return w.to(torch.bfloat16).to(device)


def fp8_weight(out_features: int, in_features: int, seed: int = 0,
               device="cpu"):
    """Random E4M3 weight codes [out_features, in_features] (uint8) and fp32
    row scales [out_features].  Codes: random sign, exponent field 3..8 and
    mantissa (magnitudes 2^-4 .. 1.875 * 2, never NaN); scales U(0.5, 1.5)
    * 2^-6, so weights are of order 1e-2."""
    import numpy as np
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, (out_features, in_features)) << 7
    e = rng.integers(3, 9, (out_features, in_features)) << 3
    m = rng.integers(0, 8, (out_features, in_features))
    codes = (sign | e | m).astype(np.uint8)
    scale = (rng.uniform(0.5, 1.5, out_features) * 2.0 ** -6).astype(np.float32)
    return (torch.from_numpy(codes).to(device),
            torch.from_numpy(scale).to(device))


def mxfp4_weight(out_features: int, in_features: int, seed: int = 0,
                 device="cpu"):
    """Random MXFP4 weight: packed E2M1 codes [out_features, in_features / 2]
    (uint8, all 16 codes equally likely) and E8M0 block scales
    [out_features, in_features / 32] drawn from 120..124 (2^-7 .. 2^-3)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (out_features, in_features // 2),
                          dtype=np.uint8)
    scales = rng.integers(120, 125, (out_features, in_features // 32),
                          dtype=np.uint8)
    return (torch.from_numpy(packed).to(device),
            torch.from_numpy(scales).to(device))
