"""ctypes wrapper of the fp64 CPU oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the CPU
baseline leg of ``bench.py``; never by the library or its binding.  The oracle
is the token-by-token gated delta rule in double precision (see the header of
``gdn_oracle.c`` for the formula and the passages it follows).

Every function takes numpy arrays or torch CPU tensors, converts them to
contiguous float64 (bf16 and fp32 values are exact in fp64), and returns
float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GATES_RAW = 0
GATES_DIRECT = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (fp64, OpenMP).  Returns its path."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O3", "-march=native", "-fopenmp", "-fPIC", "-shared",
            "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        _lib = _load_path(build())
    return _lib


def _load_path(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.gdn_oracle_prefill.argtypes = [i32, P, i32, i32, i32, i32, i32,
                                       P, P, P, P, P, P, P, P, P, P, i32]
    lib.gdn_oracle_prefill.restype = i32
    lib.gdn_oracle_decode.argtypes = [i32, i32, i32, i32, i32, i32,
                                      P, P, P, P, P, P, P, P, P, i32]
    lib.gdn_oracle_decode.restype = i32
    lib.gdn_oracle_gated_rmsnorm.argtypes = [i64, i32, P, P, P, f64, P]
    lib.gdn_oracle_gated_rmsnorm.restype = None
    lib.gdn_oracle_gates.argtypes = [i64, i32, P, P, f64, f64, P, P]
    lib.gdn_oracle_gates.restype = None
    lib.gdn_oracle_max_threads.argtypes = []
    lib.gdn_oracle_max_threads.restype = i32
    return lib


class use_library:
    """Context manager that points this wrapper at another build of the
    oracle (the mutation test compiles deliberately broken copies of
    ``gdn_oracle.c`` and checks that the pins reject each of them)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = None
        lib = _load_path(self.path)
        _lib = lib
        return lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _mode(gate_mode):
    if gate_mode in ("raw", GATES_RAW):
        return GATES_RAW
    if gate_mode in ("direct", GATES_DIRECT):
        return GATES_DIRECT
    raise ValueError("gate_mode must be 'raw' or 'direct'")


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def gates(g, beta, A_log=0.0, dt_bias=0.0, gate_mode="raw"):
    """Decay a and write strength b for 1-D arrays g, beta of one head."""
    g, beta = _f64(g).ravel(), _f64(beta).ravel()
    a = np.empty_like(g)
    b = np.empty_like(g)
    _load().gdn_oracle_gates(g.size, _mode(gate_mode), _ptr(g), _ptr(beta),
                             float(A_log), float(dt_bias), _ptr(a), _ptr(b))
    return a, b


def prefill(q, k, v, g, beta, A_log=None, dt_bias=None, *, cu_seqlens=None,
            initial_state=None, gate_mode="raw", n_threads=0,
            want_final=True):
    """Token-by-token recurrence over packed sequences.

    q, k: [T, h_k, d_k]; v: [T, h_v, d_v]; g, beta: [T, h_v];
    A_log, dt_bias: [h_v]; cu_seqlens: [N+1] (None = one sequence);
    initial_state: [N, h_v, d_v, d_k] or None (zeros).
    Returns (o [T, h_v, d_v], final_state [N, h_v, d_v, d_k] or None).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, h_k, d_k = q.shape
    _, h_v, d_v = v.shape
    mode = _mode(gate_mode)
    if mode == GATES_RAW:
        A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    else:
        A_log = dt_bias = None
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
    n = cu.size - 1
    s0 = _f64(initial_state)
    o = np.zeros((T, h_v, d_v))
    fin = np.zeros((n, h_v, d_v, d_k)) if want_final else None
    rc = _load().gdn_oracle_prefill(
        n, _ptr(cu), h_k, h_v, d_k, d_v, mode, _ptr(q), _ptr(k), _ptr(v),
        _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(s0), _ptr(fin),
        _ptr(o), int(n_threads))
    if rc != 0:
        raise ValueError("oracle prefill: bad shapes")
    return o, fin


def decode(q, k, v, g, beta, A_log, dt_bias, state, *, gate_mode="raw",
           n_threads=0):
    """One token per sequence.  q, k: [N, h_k, d_k]; v: [N, h_v, d_v];
    g, beta: [N, h_v]; state: [N, h_v, d_v, d_k].
    Returns (o [N, h_v, d_v], new_state) -- the input state is not modified."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    n, h_k, d_k = q.shape
    _, h_v, d_v = v.shape
    mode = _mode(gate_mode)
    if mode == GATES_RAW:
        A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    else:
        A_log = dt_bias = None
    st = _f64(state).copy()
    o = np.zeros((n, h_v, d_v))
    rc = _load().gdn_oracle_decode(
        n, h_k, h_v, d_k, d_v, mode, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(st), _ptr(o),
        int(n_threads))
    if rc != 0:
        raise ValueError("oracle decode: bad shapes")
    return o, st


def gated_rmsnorm(x, z, w, eps=1e-6):
    """Row-wise gated RMSNorm over the last axis: x, z [..., d], w [d]."""
    x, z, w = _f64(x), _f64(z), _f64(w)
    d = x.shape[-1]
    out = np.empty_like(x)
    _load().gdn_oracle_gated_rmsnorm(x.size // d, d, _ptr(x), _ptr(z), _ptr(w),
                                     float(eps), _ptr(out))
    return out


def tail(o, z, w, eps=1e-6):
    """Tail of the layer on a recurrent output o [T, h_v, d_v]: per-head gated
    RMSNorm, flattened head-major to [T, h_v * d_v]."""
    y = gated_rmsnorm(o, z, w, eps)
    return y.reshape(y.shape[0], -1)
