"""Thin ctypes binding over libgdn.so (C ABI in include/gdn.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory (outputs and workspace are allocated
with torch on the inputs' device) and the current HIP stream.  There is no
fallback: if libgdn.so is missing or a call fails, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK = 0
GDN_E_NULL = 1
GDN_E_SHAPE = 2
GDN_E_DTYPE = 3
GDN_E_UNSUPPORTED = 4
GDN_E_ALIGN = 5
GDN_E_WORKSPACE = 6
GDN_E_HIP = 7
GDN_E_STRUCT = 8
GDN_E_ALIAS = 9
GDN_E_SCRATCH = 10
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES

GDN_F32 = 0
GDN_BF16 = 1
GDN_GATES_RAW = 0
GDN_GATES_DIRECT = 1
GDN_WEIGHT_BF16 = 0
GDN_WEIGHT_Q4K = 1
GDN_WEIGHT_FP8 = 2
GDN_WEIGHT_MXFP4 = 3
_WEIGHT_FORMATS = {"bf16": GDN_WEIGHT_BF16, "q4k": GDN_WEIGHT_Q4K,
                   "fp8": GDN_WEIGHT_FP8, "mxfp4": GDN_WEIGHT_MXFP4}

_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("num_seqs", _i32), ("total_tokens", _i64),
        ("cu_seqlens", _P), ("cu_seqlens_host", _P),
        ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32),
        ("chunk", _i32), ("io_dtype", _i32), ("out_dtype", _i32),
        ("gate_mode", _i32),
        ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
        ("A_log", _P), ("dt_bias", _P), ("initial_state", _P),
        ("final_state", _P), ("z", _P), ("norm_weight", _P), ("eps", _f32),
        ("out", _P),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("num_seqs", _i32), ("h_k", _i32),
        ("h_v", _i32), ("d_k", _i32), ("d_v", _i32), ("io_dtype", _i32),
        ("out_dtype", _i32), ("gate_mode", _i32),
        ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
        ("A_log", _P), ("dt_bias", _P), ("state", _P), ("z", _P),
        ("norm_weight", _P), ("eps", _f32), ("out", _P),
    ]


class DecodeTokensArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("num_seqs", _i32), ("tokens_per_seq", _i32),
        ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32),
        ("io_dtype", _i32), ("out_dtype", _i32), ("gate_mode", _i32),
        ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
        ("A_log", _P), ("dt_bias", _P), ("state", _P),
        ("state_snapshots", _P), ("z", _P), ("norm_weight", _P),
        ("eps", _f32), ("out", _P),
    ]


class PrologueArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("num_seqs", _i32), ("total_tokens", _i64),
        ("cu_seqlens", _P), ("cu_seqlens_host", _P),
        ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32),
        ("width", _i32), ("io_dtype", _i32), ("out_dtype", _i32),
        ("x", _P), ("weight", _P), ("bias", _P),
        ("initial_conv_state", _P), ("final_conv_state", _P), ("eps", _f32),
        ("q", _P), ("k", _P), ("v", _P),
    ]


class RmsnormArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("d", _i32), ("rows", _i64),
        ("x_dtype", _i32), ("z_dtype", _i32), ("out_dtype", _i32),
        ("x", _P), ("z", _P), ("weight", _P), ("eps", _f32), ("out", _P),
    ]


class OutProjArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("in_features", _i32), ("rows", _i64),
        ("out_features", _i32), ("x_dtype", _i32), ("out_dtype", _i32),
        ("weight_format", _i32), ("x", _P), ("weight", _P),
        ("weight_scale", _P), ("out", _P),
    ]


class QuantArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _u32), ("format", _i32), ("rows", _i64),
        ("cols", _i32), ("x_dtype", _i32), ("x", _P), ("codes", _P),
        ("scales", _P),
    ]


_lib = None


def lib():
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libgdn.so is not built (%s); run __graft_entry__.build()"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_abi_version.restype = _u32
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_status_str.argtypes = [ctypes.c_int]
        for name, st in (("prefill", PrefillArgs), ("decode", DecodeArgs),
                         ("decode_tokens", DecodeTokensArgs),
                         ("prologue", PrologueArgs),
                         ("rmsnorm", RmsnormArgs),
                         ("out_proj", OutProjArgs),
                         ("quantize_act", QuantArgs)):
            f = getattr(L, "gdn_validate_" + name)
            f.argtypes = [ctypes.POINTER(st)]
            f.restype = ctypes.c_int
        L.gdn_prefill_workspace_size.argtypes = [
            ctypes.POINTER(PrefillArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_prefill_workspace_size.restype = ctypes.c_int
        L.gdn_chunk_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _P,
                                        ctypes.c_size_t, _P]
        L.gdn_chunk_prefill.restype = ctypes.c_int
        L.gdn_chunk_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _P]
        L.gdn_chunk_prefill_noalloc.restype = ctypes.c_int
        L.gdn_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _P]
        L.gdn_decode_step.restype = ctypes.c_int
        L.gdn_decode_tokens.argtypes = [ctypes.POINTER(DecodeTokensArgs), _P]
        L.gdn_decode_tokens.restype = ctypes.c_int
        L.gdn_conv_prologue.argtypes = [ctypes.POINTER(PrologueArgs), _P]
        L.gdn_conv_prologue.restype = ctypes.c_int
        L.gdn_gated_rmsnorm.argtypes = [ctypes.POINTER(RmsnormArgs), _P]
        L.gdn_gated_rmsnorm.restype = ctypes.c_int
        L.gdn_out_proj_workspace_size.argtypes = [
            ctypes.POINTER(OutProjArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.gdn_out_proj_workspace_size.restype = ctypes.c_int
        L.gdn_out_proj.argtypes = [ctypes.POINTER(OutProjArgs), _P,
                                   ctypes.c_size_t, _P]
        L.gdn_out_proj.restype = ctypes.c_int
        L.gdn_quantize_act.argtypes = [ctypes.POINTER(QuantArgs), _P]
        L.gdn_quantize_act.restype = ctypes.c_int
        _lib = L
    return _lib


def gdn_abi_version() -> int:
    return int(lib().gdn_abi_version())


def gdn_status_str(status: int) -> str:
    return lib().gdn_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != GDN_OK:
        raise RuntimeError("%s failed: %s (code %d)" % (
            what, gdn_status_str(status), status))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == GDN_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(t, name, device, dtype=None, shape=None):
    """Marshalling check of one tensor argument: it must live on `device`,
    and have `dtype` and `shape` when those are given (None entries of
    `shape` match any size).  The library sees raw pointers only, so a
    tensor of another dtype or device would be read as garbage."""
    if t is None:
        return
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None:
        ok = t.dim() == len(shape) and all(
            s is None or int(n) == int(s) for n, s in zip(t.shape, shape))
        if not ok:
            raise ValueError("%s has shape %s, expected %s" % (
                name, tuple(t.shape),
                tuple("*" if s is None else s for s in shape)))


def _check_layer_tensors(q, k, v, g, beta, A_log, dt_bias, z, norm_weight,
                         cu_seqlens, states, rows):
    """Device / dtype / shape checks shared by the prefill and decode
    calls: q, k, v, z in one io dtype (fp32 or bf16); gates, gate
    parameters, norm weight and states fp32; cu_seqlens int32 [N+1]; every
    tensor on q's device.  `rows` is the token count the gates and v must
    have; `states` maps names to (tensor, expected shape)."""
    dev = q.device
    io = q.dtype
    _dt(q)
    T, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    _expect(k, "k", dev, io, (T, h_k, d_k))
    _expect(v, "v", dev, io, (rows, h_v, d_v))
    _expect(z, "z", dev, io, (rows, h_v, d_v))
    _expect(g, "g", dev, torch.float32, (rows, h_v))
    _expect(beta, "beta", dev, torch.float32, (rows, h_v))
    _expect(A_log, "A_log", dev, torch.float32, (h_v,))
    _expect(dt_bias, "dt_bias", dev, torch.float32, (h_v,))
    _expect(norm_weight, "norm_weight", dev, torch.float32, (d_v,))
    _expect(cu_seqlens, "cu_seqlens", dev, torch.int32, (None,))
    for name, (t, shape) in states.items():
        _expect(t, name, dev, torch.float32, shape)


def _stream(device: torch.device):
    if device.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    return torch.cuda.current_stream(device).cuda_stream


def _gate_mode(mode) -> int:
    if mode in ("raw", GDN_GATES_RAW):
        return GDN_GATES_RAW
    if mode in ("direct", GDN_GATES_DIRECT):
        return GDN_GATES_DIRECT
    raise ValueError("gate_mode must be 'raw' or 'direct'")


def make_prefill_args(q, k, v, g, beta, A_log=None, dt_bias=None, *,
                      cu_seqlens=None, cu_seqlens_host=None, num_seqs=None,
                      initial_state=None, final_state=None, z=None,
                      norm_weight=None, eps=1e-6, chunk_size=64,
                      gate_mode="raw", out=None, out_dtype=None):
    """Fill a PrefillArgs from tensors (no allocation, no launch).  Returns
    (args, keepalive) -- keep the second value alive while args is used."""
    T, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if num_seqs is None:
        num_seqs = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    a = PrefillArgs()
    a.struct_size = ctypes.sizeof(PrefillArgs)
    a.num_seqs = int(num_seqs)
    a.total_tokens = int(T)
    a.cu_seqlens = _ptr(cu_seqlens)
    host = None
    if cu_seqlens_host is not None:
        host = (ctypes.c_int32 * len(cu_seqlens_host))(
            *[int(x) for x in cu_seqlens_host])
        a.cu_seqlens_host = ctypes.cast(host, _P)
    a.h_k, a.h_v, a.d_k, a.d_v = int(h_k), int(h_v), int(d_k), int(d_v)
    a.chunk = int(chunk_size)
    a.io_dtype = _dt(q)
    a.out_dtype = out_dtype if out_dtype is not None else a.io_dtype
    a.gate_mode = _gate_mode(gate_mode)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.g, a.beta = _ptr(g), _ptr(beta)
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.initial_state, a.final_state = _ptr(initial_state), _ptr(final_state)
    a.z, a.norm_weight = _ptr(z), _ptr(norm_weight)
    a.eps = float(eps)
    a.out = _ptr(out)
    return a, host


def gdn_prefill_workspace_size(args: PrefillArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_prefill_workspace_size(ctypes.byref(args),
                                            ctypes.byref(n)),
           "gdn_prefill_workspace_size")
    return int(n.value)


def gdn_chunk_prefill(q, k, v, g, beta, A_log=None, dt_bias=None, *,
                      cu_seqlens=None, cu_seqlens_host=None,
                      initial_state=None, output_final_state=True,
                      final_state=None, z=None, norm_weight=None, eps=1e-6,
                      chunk_size=64, gate_mode="raw", out_dtype=None,
                      out=None, workspace=None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill.  q, k: [T, h_k, d_k]; v, z: [T, h_v, d_v];
    g, beta: [T, h_v] fp32; A_log, dt_bias: [h_v] fp32; cu_seqlens: int32
    [N+1] on the device.  Returns (out, final_state): out is o [T, h_v, d_v]
    or, with z, the gated RMSNorm [T, h_v * d_v]."""
    T, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = q.device
    if cu_seqlens is not None and cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs N+1 >= 2 offsets")
    if cu_seqlens_host is not None and len(cu_seqlens_host) != n + 1:
        raise ValueError("cu_seqlens_host has %d offsets, expected %d"
                         % (len(cu_seqlens_host), n + 1))
    _check_layer_tensors(q, k, v, g, beta, A_log, dt_bias, z, norm_weight,
                         cu_seqlens, {
                             "initial_state": (initial_state, (n, h_v, d_v, d_k)),
                             "final_state": (final_state, (n, h_v, d_v, d_k))},
                         T)
    odt = _dt(q) if out_dtype is None else (
        out_dtype if isinstance(out_dtype, int) else _dt(
            torch.empty(0, dtype=out_dtype)))
    shape = (T, h_v * d_v) if z is not None else (T, h_v, d_v)
    if out is None:
        out = torch.empty(shape, dtype=_torch_dtype(odt), device=dev)
    _expect(out, "out", dev, _torch_dtype(odt), shape)
    _expect(workspace, "workspace", dev)
    if final_state is None and output_final_state:
        final_state = torch.empty(n, h_v, d_v, d_k, dtype=torch.float32,
                                  device=dev)
    a, keep = make_prefill_args(
        q, k, v, g, beta, A_log, dt_bias, cu_seqlens=cu_seqlens,
        cu_seqlens_host=cu_seqlens_host, num_seqs=n,
        initial_state=initial_state, final_state=final_state, z=z,
        norm_weight=norm_weight, eps=eps, chunk_size=chunk_size,
        gate_mode=gate_mode, out=out, out_dtype=odt)
    ws_bytes = gdn_prefill_workspace_size(a)
    if ws_bytes and (workspace is None or workspace.numel() *
                     workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace) if ws_bytes else None
    _check(lib().gdn_chunk_prefill(ctypes.byref(a), ws_ptr, ws_bytes,
                                   _stream(dev)), "gdn_chunk_prefill")
    del keep
    return out, final_state


def gdn_chunk_prefill_noalloc(q, k, v, g, beta, A_log=None, dt_bias=None, *,
                              out, cu_seqlens=None, cu_seqlens_host=None,
                              initial_state=None, final_state=None, z=None,
                              norm_weight=None, eps=1e-6, chunk_size=64,
                              gate_mode="raw"):
    """gdn_chunk_prefill on the library's static per-GPU scratch: nothing is
    allocated, so `out` (and `final_state`, when wanted) must be passed;
    their dtypes and shapes are those gdn_chunk_prefill returns.  Calls that
    overlap in time on one GPU race on the shared scratch."""
    T, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = q.device
    if cu_seqlens is not None and cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs N+1 >= 2 offsets")
    if cu_seqlens_host is not None and len(cu_seqlens_host) != n + 1:
        raise ValueError("cu_seqlens_host has %d offsets, expected %d"
                         % (len(cu_seqlens_host), n + 1))
    _check_layer_tensors(q, k, v, g, beta, A_log, dt_bias, z, norm_weight,
                         cu_seqlens, {
                             "initial_state": (initial_state, (n, h_v, d_v, d_k)),
                             "final_state": (final_state, (n, h_v, d_v, d_k))},
                         T)
    if out is None:
        raise ValueError("out is required (this call allocates nothing)")
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16, got %s" % out.dtype)
    shape = (T, h_v * d_v) if z is not None else (T, h_v, d_v)
    _expect(out, "out", dev, out.dtype, shape)
    a, keep = make_prefill_args(
        q, k, v, g, beta, A_log, dt_bias, cu_seqlens=cu_seqlens,
        cu_seqlens_host=cu_seqlens_host, num_seqs=n,
        initial_state=initial_state, final_state=final_state, z=z,
        norm_weight=norm_weight, eps=eps, chunk_size=chunk_size,
        gate_mode=gate_mode, out=out, out_dtype=_dt(out))
    _check(lib().gdn_chunk_prefill_noalloc(ctypes.byref(a), _stream(dev)),
           "gdn_chunk_prefill_noalloc")
    del keep
    return out, final_state


def make_decode_args(q, k, v, g, beta, A_log, dt_bias, state, *, z=None,
                     norm_weight=None, eps=1e-6, gate_mode="raw", out=None,
                     out_dtype=None):
    N, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    a.num_seqs, a.h_k, a.h_v, a.d_k, a.d_v = N, h_k, h_v, d_k, d_v
    a.io_dtype = _dt(q)
    a.out_dtype = out_dtype if out_dtype is not None else a.io_dtype
    a.gate_mode = _gate_mode(gate_mode)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.g, a.beta = _ptr(g), _ptr(beta)
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.state = _ptr(state)
    a.z, a.norm_weight = _ptr(z), _ptr(norm_weight)
    a.eps = float(eps)
    a.out = _ptr(out)
    return a


def gdn_decode_step(q, k, v, g, beta, A_log, dt_bias, state, *, z=None,
                    norm_weight=None, eps=1e-6, gate_mode="raw",
                    out_dtype=None, out=None) -> torch.Tensor:
    """One decode step; `state` [N, h_v, d_v, d_k] fp32 is updated in place.
    Returns o [N, h_v, d_v] or, with z, the gated RMSNorm [N, h_v * d_v]."""
    N, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    _check_layer_tensors(q, k, v, g, beta, A_log, dt_bias, z, norm_weight,
                         None, {"state": (state, (N, h_v, d_v, d_k))}, N)
    odt = _dt(q) if out_dtype is None else (
        out_dtype if isinstance(out_dtype, int) else _dt(
            torch.empty(0, dtype=out_dtype)))
    shape = (N, h_v * d_v) if z is not None else (N, h_v, d_v)
    if out is None:
        out = torch.empty(shape, dtype=_torch_dtype(odt), device=q.device)
    _expect(out, "out", q.device, _torch_dtype(odt), shape)
    a = make_decode_args(q, k, v, g, beta, A_log, dt_bias, state, z=z,
                         norm_weight=norm_weight, eps=eps, gate_mode=gate_mode,
                         out=out, out_dtype=odt)
    _check(lib().gdn_decode_step(ctypes.byref(a), _stream(q.device)),
           "gdn_decode_step")
    return out


def make_decode_tokens_args(q, k, v, g, beta, A_log, dt_bias, state, *,
                            tokens_per_seq, snapshots=None, z=None,
                            norm_weight=None, eps=1e-6, gate_mode="raw",
                            out=None, out_dtype=None):
    NT, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    N = state.shape[0]
    a = DecodeTokensArgs()
    a.struct_size = ctypes.sizeof(DecodeTokensArgs)
    a.num_seqs, a.tokens_per_seq = N, int(tokens_per_seq)
    a.h_k, a.h_v, a.d_k, a.d_v = h_k, h_v, d_k, d_v
    a.io_dtype = _dt(q)
    a.out_dtype = out_dtype if out_dtype is not None else a.io_dtype
    a.gate_mode = _gate_mode(gate_mode)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.g, a.beta = _ptr(g), _ptr(beta)
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.state = _ptr(state)
    a.state_snapshots = _ptr(snapshots)
    a.z, a.norm_weight = _ptr(z), _ptr(norm_weight)
    a.eps = float(eps)
    a.out = _ptr(out)
    return a


def gdn_decode_tokens(q, k, v, g, beta, A_log, dt_bias, state, *,
                      tokens_per_seq, snapshots=False, z=None,
                      norm_weight=None, eps=1e-6, gate_mode="raw",
                      out_dtype=None, out=None):
    """T = tokens_per_seq decode tokens for each of the N sequences of
    `state` [N, h_v, d_v, d_k] fp32 (updated in place to the state after the
    last token).  q, k: [N*T, h_k, d_k]; v, z: [N*T, h_v, d_v]; g, beta:
    [N*T, h_v]; row n*T + t is token t of sequence n.  With snapshots=True
    (or a [N, T, h_v, d_v, d_k] fp32 tensor) the state after every token is
    returned too.  Returns (out, snapshots or None)."""
    NT, h_k, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    N = state.shape[0]
    T = int(tokens_per_seq)
    if NT != N * T:
        raise ValueError("q has %d rows, expected N*T = %d" % (NT, N * T))
    _check_layer_tensors(q, k, v, g, beta, A_log, dt_bias, z, norm_weight,
                         None, {"state": (state, (N, h_v, d_v, d_k))}, NT)
    if isinstance(snapshots, torch.Tensor):
        _expect(snapshots, "snapshots", q.device, torch.float32,
                (N, T, h_v, d_v, d_k))
    odt = _dt(q) if out_dtype is None else (
        out_dtype if isinstance(out_dtype, int) else _dt(
            torch.empty(0, dtype=out_dtype)))
    shape = (NT, h_v * d_v) if z is not None else (NT, h_v, d_v)
    if out is None:
        out = torch.empty(shape, dtype=_torch_dtype(odt), device=q.device)
    _expect(out, "out", q.device, _torch_dtype(odt), shape)
    snaps = None
    if snapshots is True:
        snaps = torch.empty((N, T, h_v, d_v, d_k), dtype=torch.float32,
                            device=q.device)
    elif isinstance(snapshots, torch.Tensor):
        snaps = snapshots
    a = make_decode_tokens_args(q, k, v, g, beta, A_log, dt_bias, state,
                                tokens_per_seq=T, snapshots=snaps, z=z,
                                norm_weight=norm_weight, eps=eps,
                                gate_mode=gate_mode, out=out, out_dtype=odt)
    _check(lib().gdn_decode_tokens(ctypes.byref(a), _stream(q.device)),
           "gdn_decode_tokens")
    return out, snaps


def make_prologue_args(x, weight, bias, *, h_k, h_v, d_k, d_v,
                       cu_seqlens=None, cu_seqlens_host=None,
                       initial_conv_state=None, final_conv_state=None,
                       eps=1e-6, q=None, k=None, v=None, out_dtype=None):
    """Argument struct and the host arrays it points into (keep them alive
    for the duration of the call)."""
    T = x.shape[0]
    a = PrologueArgs()
    a.struct_size = ctypes.sizeof(PrologueArgs)
    keep = []
    if cu_seqlens is None:
        a.num_seqs = 1
    else:
        a.num_seqs = int(cu_seqlens.numel()) - 1
    a.total_tokens = int(T)
    a.cu_seqlens = _ptr(cu_seqlens)
    if cu_seqlens_host is not None:
        h = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(c) for c in cu_seqlens_host])
        keep.append(h)
        a.cu_seqlens_host = ctypes.cast(h, ctypes.c_void_p)
    a.h_k, a.h_v, a.d_k, a.d_v = h_k, h_v, d_k, d_v
    a.width = int(weight.shape[1])
    a.io_dtype = _dt(x)
    a.out_dtype = out_dtype if out_dtype is not None else a.io_dtype
    a.x, a.weight, a.bias = _ptr(x), _ptr(weight), _ptr(bias)
    a.initial_conv_state = _ptr(initial_conv_state)
    a.final_conv_state = _ptr(final_conv_state)
    a.eps = float(eps)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    return a, keep


def gdn_conv_prologue(x, weight, bias=None, *, h_k, h_v, d_k, d_v,
                      cu_seqlens=None, cu_seqlens_host=None,
                      initial_conv_state=None, output_final_state=False,
                      final_conv_state=None, eps=1e-6, out_dtype=None,
                      q=None, k=None, v=None):
    """Causal convolution (+ SiLU) over x [T, C] (C = 2 h_k d_k + h_v d_v
    channels: q, k, v) within each packed sequence, then per-head L2
    normalization of q and k.  weight [C, W] fp32, bias [C] fp32 or None,
    conv states [N, C, W-1] fp32.  Returns (q, k, v, final_conv_state)."""
    T = x.shape[0]
    W = int(weight.shape[1])
    odt = _dt(x) if out_dtype is None else (
        out_dtype if isinstance(out_dtype, int) else _dt(
            torch.empty(0, dtype=out_dtype)))
    tdt = _torch_dtype(odt)
    if q is None:
        q = torch.empty(T, h_k, d_k, dtype=tdt, device=x.device)
    if k is None:
        k = torch.empty(T, h_k, d_k, dtype=tdt, device=x.device)
    if v is None:
        v = torch.empty(T, h_v, d_v, dtype=tdt, device=x.device)
    N = 1 if cu_seqlens is None else int(cu_seqlens.numel()) - 1
    C = 2 * h_k * d_k + h_v * d_v
    dev = x.device
    _dt(x)
    _expect(x, "x", dev, None, (T, C))
    _expect(weight, "weight", dev, torch.float32, (C, W))
    _expect(bias, "bias", dev, torch.float32, (C,))
    _expect(cu_seqlens, "cu_seqlens", dev, torch.int32, (None,))
    if cu_seqlens is not None and cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs N+1 >= 2 offsets")
    _expect(initial_conv_state, "initial_conv_state", dev, torch.float32,
            (N, C, W - 1))
    _expect(final_conv_state, "final_conv_state", dev, torch.float32,
            (N, C, W - 1))
    for name, t, shape in (("q", q, (T, h_k, d_k)), ("k", k, (T, h_k, d_k)),
                           ("v", v, (T, h_v, d_v))):
        _expect(t, name, dev, tdt, shape)
    if output_final_state and final_conv_state is None:
        final_conv_state = torch.empty(N, C, W - 1, dtype=torch.float32,
                                       device=x.device)
    a, keep = make_prologue_args(
        x, weight, bias, h_k=h_k, h_v=h_v, d_k=d_k, d_v=d_v,
        cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host,
        initial_conv_state=initial_conv_state,
        final_conv_state=final_conv_state, eps=eps, q=q, k=k, v=v,
        out_dtype=odt)
    _check(lib().gdn_conv_prologue(ctypes.byref(a), _stream(x.device)),
           "gdn_conv_prologue")
    del keep
    return q, k, v, final_conv_state


def make_rmsnorm_args(x, z, weight, eps=1e-6, out=None, out_dtype=None):
    d = x.shape[-1]
    a = RmsnormArgs()
    a.struct_size = ctypes.sizeof(RmsnormArgs)
    a.d = int(d)
    a.rows = int(x.numel() // d) if d else 0
    a.x_dtype, a.z_dtype = _dt(x), _dt(z)
    a.out_dtype = out_dtype if out_dtype is not None else a.x_dtype
    a.x, a.z, a.weight = _ptr(x), _ptr(z), _ptr(weight)
    a.eps = float(eps)
    a.out = _ptr(out)
    return a


def gdn_gated_rmsnorm(x, z, weight, eps=1e-6, *, out_dtype=None,
                      out=None) -> torch.Tensor:
    """Standalone gated RMSNorm over the last axis of x (and z)."""
    odt = _dt(x) if out_dtype is None else (
        out_dtype if isinstance(out_dtype, int) else _dt(
            torch.empty(0, dtype=out_dtype)))
    if out is None:
        out = torch.empty(x.shape, dtype=_torch_dtype(odt), device=x.device)
    _dt(z)
    _expect(z, "z", x.device, None, tuple(x.shape))
    _expect(weight, "weight", x.device, torch.float32, (x.shape[-1],))
    _expect(out, "out", x.device, _torch_dtype(odt), tuple(x.shape))
    a = make_rmsnorm_args(x, z, weight, eps, out=out, out_dtype=odt)
    _check(lib().gdn_gated_rmsnorm(ctypes.byref(a), _stream(x.device)),
           "gdn_gated_rmsnorm")
    return out


def _wfmt(q4k, weight_format):
    if weight_format is None:
        return GDN_WEIGHT_Q4K if q4k else GDN_WEIGHT_BF16
    if isinstance(weight_format, str):
        return _WEIGHT_FORMATS[weight_format]
    return int(weight_format)


def make_out_proj_args(x, weight, out_features, *, q4k=False,
                       weight_format=None, weight_scale=None, out=None,
                       out_dtype=None):
    """x: [M, K]; weight: bf16 [N, K], uint8 Q4_K bytes (N * K / 256 blocks
    of 144), uint8 E4M3 codes [N, K] with fp32 weight_scale [N], or uint8
    packed E2M1 codes [N, K / 2] with uint8 E8M0 weight_scale [N, K / 32]."""
    a = OutProjArgs()
    a.struct_size = ctypes.sizeof(OutProjArgs)
    a.rows = int(x.shape[0])
    a.in_features = int(x.shape[1])
    a.out_features = int(out_features)
    a.x_dtype = _dt(x)
    a.out_dtype = out_dtype if out_dtype is not None else a.x_dtype
    a.weight_format = _wfmt(q4k, weight_format)
    a.x, a.weight, a.out = _ptr(x), _ptr(weight), _ptr(out)
    a.weight_scale = _ptr(weight_scale)
    return a


def gdn_out_proj_workspace_size(args: OutProjArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_out_proj_workspace_size(ctypes.byref(args),
                                             ctypes.byref(n)),
           "gdn_out_proj_workspace_size")
    return int(n.value)


def gdn_out_proj(x, weight, out_features=None, *, q4k=False,
                 weight_format=None, weight_scale=None, out_dtype=None,
                 out=None, workspace=None) -> torch.Tensor:
    """Output projection out = x W^T (W [out_features, in_features]: dense
    bf16, packed Q4_K, or E4M3 / MXFP4 codes with their scales, the
    activations then quantized on the GPU)."""
    fmt = _wfmt(q4k, weight_format)
    if out_features is None:
        if fmt in (GDN_WEIGHT_Q4K, GDN_WEIGHT_MXFP4):
            raise ValueError("out_features is required for a packed weight")
        out_features = int(weight.shape[0])
    odt = _dt(x) if out_dtype is None else (
        out_dtype if isinstance(out_dtype, int) else _dt(
            torch.empty(0, dtype=out_dtype)))
    if out is None:
        out = torch.empty(x.shape[0], int(out_features),
                          dtype=_torch_dtype(odt), device=x.device)
    _dt(x)
    _expect(out, "out", x.device, _torch_dtype(odt),
            (x.shape[0], int(out_features)))
    _expect(weight, "weight", x.device,
            torch.bfloat16 if fmt == GDN_WEIGHT_BF16 else torch.uint8)
    _expect(weight_scale, "weight_scale", x.device,
            torch.float32 if fmt == GDN_WEIGHT_FP8 else torch.uint8)
    _expect(workspace, "workspace", x.device)
    a = make_out_proj_args(x, weight, out_features, weight_format=fmt,
                           weight_scale=weight_scale, out=out, out_dtype=odt)
    need = gdn_out_proj_workspace_size(a)
    if need and (workspace is None or workspace.numel() *
                 workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else (workspace.numel() *
                                            workspace.element_size())
    _check(lib().gdn_out_proj(ctypes.byref(a), _ptr(workspace), ws_bytes,
                              _stream(x.device)), "gdn_out_proj")
    return out


def make_quant_args(x, fmt, codes, scales):
    a = QuantArgs()
    a.struct_size = ctypes.sizeof(QuantArgs)
    a.format = _wfmt(False, fmt)
    a.rows = int(x.shape[0])
    a.cols = int(x.shape[1])
    a.x_dtype = _dt(x)
    a.x, a.codes, a.scales = _ptr(x), _ptr(codes), _ptr(scales)
    return a


def gdn_quantize_act(x, fmt="fp8"):
    """Activation quantization of the FP8 / MXFP4 projections: returns
    (codes, scales) -- FP8: uint8 [M, K] and fp32 [M]; MXFP4: uint8
    [M, K / 2] and uint8 [M, K / 32]."""
    M, K = int(x.shape[0]), int(x.shape[1])
    if _wfmt(False, fmt) == GDN_WEIGHT_FP8:
        codes = torch.empty(M, K, dtype=torch.uint8, device=x.device)
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    else:
        codes = torch.empty(M, K // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(M, K // 32, dtype=torch.uint8, device=x.device)
    a = make_quant_args(x, fmt, codes, scales)
    _check(lib().gdn_quantize_act(ctypes.byref(a), _stream(x.device)),
           "gdn_quantize_act")
    return codes, scales


def gdn_validate_quantize_act(args: QuantArgs) -> int:
    return int(lib().gdn_validate_quantize_act(ctypes.byref(args)))


def gdn_validate_out_proj(args: OutProjArgs) -> int:
    return int(lib().gdn_validate_out_proj(ctypes.byref(args)))


def gdn_validate_prefill(args: PrefillArgs) -> int:
    return int(lib().gdn_validate_prefill(ctypes.byref(args)))


def gdn_validate_decode(args: DecodeArgs) -> int:
    return int(lib().gdn_validate_decode(ctypes.byref(args)))


def gdn_validate_decode_tokens(args: DecodeTokensArgs) -> int:
    return int(lib().gdn_validate_decode_tokens(ctypes.byref(args)))


def gdn_validate_prologue(args: PrologueArgs) -> int:
    return int(lib().gdn_validate_prologue(ctypes.byref(args)))


def gdn_validate_rmsnorm(args: RmsnormArgs) -> int:
    return int(lib().gdn_validate_rmsnorm(ctypes.byref(args)))
