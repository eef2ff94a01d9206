"""Python access to the CPU oracle (``switch_oracle.c``) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does.  Arrays are numpy; floating inputs are float32
(bf16 inputs widen to float32 exactly before they get here), results are
float64 / int32 / uint8.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def threads() -> int:
    """Every core the process may run on (its affinity mask)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, n)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_capacity.argtypes = [_i64, _i64, ctypes.c_double, _i64]
        L.oracle_capacity.restype = _i64
        L.oracle_logits.argtypes = [_f32p, _f32p, _vp, _i64, _i64, _i64, _f64p, ctypes.c_int]
        L.oracle_logits.restype = None
        L.oracle_route.argtypes = [_f64p, _i64, _i64, ctypes.c_double, _i64, ctypes.c_double,
                                   _i32p, _f64p, _i32p, _u8p, _i32p, _f64p, _f64p, ctypes.c_int]
        L.oracle_route.restype = _i64
        L.oracle_token_output.argtypes = [_f32p, ctypes.c_int32, ctypes.c_double, _f32p, _f32p,
                                          _i64, _i64, _f64p, _f64p]
        L.oracle_token_output.restype = None
        L.oracle_combine.argtypes = [_f32p, _i32p, _f64p, _u8p, _f32p, _f32p, _i64, _i64, _i64,
                                     _f64p, _f64p, ctypes.c_int]
        L.oracle_combine.restype = None
        L.oracle_capacity_topk.argtypes = [_i64, _i64, _i64, ctypes.c_double, _i64]
        L.oracle_capacity_topk.restype = _i64
        L.oracle_route_topk.argtypes = [_f64p, _i64, _i64, _i64, ctypes.c_double, _i64,
                                        ctypes.c_double, _i32p, _f64p, _i32p, _u8p, _i32p, _f64p,
                                        _f64p, ctypes.c_int]
        L.oracle_route_topk.restype = _i64
        L.oracle_combine_topk.argtypes = [_f32p, _i32p, _f64p, _u8p, _f32p, _f32p, _i64, _i64,
                                          _i64, _i64, _f64p, _f64p, ctypes.c_int]
        L.oracle_combine_topk.restype = None
        L.oracle_backward.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _i32p, _f64p, _u8p,
                                      _i32p, _f64p, ctypes.c_double, ctypes.c_double, _i64, _i64,
                                      _i64, _i64, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int]
        L.oracle_backward.restype = None
        L.oracle_backward_topk.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _i32p, _f64p,
                                           _u8p, _i32p, _f64p, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, _f64p, _f64p, _f64p,
                                           _f64p, _f64p, ctypes.c_int]
        L.oracle_backward_topk.restype = None
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def capacity(T: int, N: int, c: float, capacity_override: int = 0) -> int:
    return int(lib().oracle_capacity(T, N, c, capacity_override))


def logits(x, W_r, b_r=None, nthreads: int = 0) -> np.ndarray:
    x = _c(x, np.float32)
    W_r = _c(W_r, np.float32)
    T, d = x.shape
    N = W_r.shape[0]
    h = np.empty((T, N), dtype=np.float64)
    b = None if b_r is None else _c(b_r, np.float32)
    lib().oracle_logits(x, W_r, None if b is None else b.ctypes.data_as(_vp), T, d, N, h,
                        nthreads or threads())
    return h


def route(h, c: float, capacity_override: int = 0, alpha: float = 0.01, nthreads: int = 0) -> dict:
    """Routing stage on given logits [T, N] (float32 logits widen exactly)."""
    h = _c(h, np.float64)
    T, N = h.shape
    r = dict(expert_idx=np.empty(T, np.int32), gate=np.empty(T, np.float64),
             position=np.empty(T, np.int32), drop=np.empty(T, np.uint8),
             load=np.empty(N, np.int32), P=np.empty(N, np.float64))
    aux = np.zeros(1, np.float64)
    C = lib().oracle_route(h, T, N, c, capacity_override, alpha, r["expert_idx"], r["gate"],
                           r["position"], r["drop"], r["load"], r["P"], aux, nthreads or threads())
    r["aux"] = float(aux[0])
    r["C"] = int(C)
    return r


def token_output(x_row, dropped: bool, gate: float, W_in_e, W_out_e):
    """(out row, expert output row) of one token."""
    x_row = _c(x_row, np.float32)
    W_in_e = _c(W_in_e, np.float32)
    W_out_e = _c(W_out_e, np.float32)
    F, d = W_in_e.shape
    out = np.empty(d, np.float64)
    E = np.empty(d, np.float64)
    lib().oracle_token_output(x_row, int(bool(dropped)), float(gate), W_in_e, W_out_e, d, F, out, E)
    return out, E


def combine(x, expert_idx, gate, drop, W_in, W_out, nthreads: int = 0):
    x = _c(x, np.float32)
    W_in = _c(W_in, np.float32)
    W_out = _c(W_out, np.float32)
    T, d = x.shape
    F = W_in.shape[1]
    out = np.empty((T, d), np.float64)
    E = np.empty((T, d), np.float64)
    lib().oracle_combine(x, _c(expert_idx, np.int32), _c(gate, np.float64), _c(drop, np.uint8),
                         W_in, W_out, T, d, F, out, E, nthreads or threads())
    return out, E


def capacity_topk(T: int, N: int, k: int, c: float, capacity_override: int = 0) -> int:
    return int(lib().oracle_capacity_topk(T, N, k, c, capacity_override))


def route_topk(h, k: int, c: float, capacity_override: int = 0, alpha: float = 0.01,
               nthreads: int = 0) -> dict:
    """Top-k routing stage on given logits [T, N]; per-choice outputs are [T, k]."""
    h = _c(h, np.float64)
    T, N = h.shape
    assert 1 <= k <= N
    r = dict(expert_idx=np.empty((T, k), np.int32), gate=np.empty((T, k), np.float64),
             position=np.empty((T, k), np.int32), drop=np.empty((T, k), np.uint8),
             load=np.empty(N, np.int32), P=np.empty(N, np.float64))
    aux = np.zeros(1, np.float64)
    C = lib().oracle_route_topk(h, T, N, k, c, capacity_override, alpha, r["expert_idx"],
                                r["gate"], r["position"], r["drop"], r["load"], r["P"], aux,
                                nthreads or threads())
    r["aux"] = float(aux[0])
    r["C"] = int(C)
    return r


def combine_topk(x, expert_idx, gate, drop, W_in, W_out, nthreads: int = 0):
    """(out [T, d], per-choice expert outputs [T, k, d])."""
    x = _c(x, np.float32)
    W_in = _c(W_in, np.float32)
    W_out = _c(W_out, np.float32)
    T, d = x.shape
    F = W_in.shape[1]
    expert_idx = _c(expert_idx, np.int32)
    k = expert_idx.shape[1]
    out = np.empty((T, d), np.float64)
    E = np.empty((T, k, d), np.float64)
    lib().oracle_combine_topk(x, expert_idx, _c(gate, np.float64), _c(drop, np.uint8), W_in,
                              W_out, T, k, d, F, out, E, nthreads or threads())
    return out, E


def forward(x, W_r, b_r, W_in, W_out, c: float, capacity_override: int = 0, alpha: float = 0.01,
            nthreads: int = 0) -> dict:
    """The whole layer in the pages' order: logits, routing, expert FFN and combine."""
    h = logits(x, W_r, b_r, nthreads)
    r = route(h, c, capacity_override, alpha, nthreads)
    out, E = combine(x, r["expert_idx"], r["gate"], r["drop"], W_in, W_out, nthreads)
    r.update(h=h, out=out, E=E)
    return r


def backward(x, W_r, W_in, W_out, h, expert_idx, gate, drop, load, G, g_aux: float = 0.0,
             alpha: float = 0.01, nthreads: int = 0) -> dict:
    """Gradients of the top-1 layer for dL/dout = G and dL/daux = g_aux, at the
    forward's routing (expert_idx, gate, drop), logits h and loads."""
    x = _c(x, np.float32)
    T, d = x.shape
    W_in = _c(W_in, np.float32)
    W_out = _c(W_out, np.float32)
    N, F = W_in.shape[0], W_in.shape[1]
    r = dict(dx=np.empty((T, d)), dW_r=np.empty((N, d)), db=np.empty(N),
             dW_in=np.empty((N, F, d)), dW_out=np.empty((N, d, F)))
    lib().oracle_backward(x, _c(W_r, np.float32), W_in, W_out, _c(h, np.float64),
                          _c(expert_idx, np.int32), _c(gate, np.float64), _c(drop, np.uint8),
                          _c(load, np.int32), _c(G, np.float64), g_aux, alpha, T, d, F, N,
                          r["dx"], r["dW_r"], r["db"], r["dW_in"], r["dW_out"],
                          nthreads or threads())
    return r


def backward_topk(x, W_r, W_in, W_out, h, expert_idx, gate, drop, load, G, g_aux: float = 0.0,
                  alpha: float = 0.01, nthreads: int = 0) -> dict:
    """Gradients of the top-k layer (expert_idx, gate, drop [T, k]) for dL/dout = G
    and dL/daux = g_aux, at the forward's routing, logits h and loads."""
    x = _c(x, np.float32)
    T, d = x.shape
    W_in = _c(W_in, np.float32)
    W_out = _c(W_out, np.float32)
    N, F = W_in.shape[0], W_in.shape[1]
    expert_idx = _c(np.asarray(expert_idx).reshape(T, -1), np.int32)
    k = expert_idx.shape[1]
    r = dict(dx=np.empty((T, d)), dW_r=np.empty((N, d)), db=np.empty(N),
             dW_in=np.empty((N, F, d)), dW_out=np.empty((N, d, F)))
    lib().oracle_backward_topk(x, _c(W_r, np.float32), W_in, W_out, _c(h, np.float64),
                               expert_idx, _c(np.asarray(gate).reshape(T, k), np.float64),
                               _c(np.asarray(drop).reshape(T, k), np.uint8), _c(load, np.int32),
                               _c(G, np.float64), g_aux, alpha, T, k, d, F, N, r["dx"],
                               r["dW_r"], r["db"], r["dW_in"], r["dW_out"], nthreads or threads())
    return r
