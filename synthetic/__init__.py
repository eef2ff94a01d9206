"""Seeded synthetic inputs for the Switch FFN layer (shared by the HIP tests,
the benchmark and the CPU oracle).

This package draws numbers and nothing else: it holds none of the layer's
arithmetic (no routing, capacity, softmax or FFN).  The counter-based
definition lives in ``synth.c`` (host) and ``synth_gpu.hip`` (device, for
weight banks too large to stage through host memory).

Workload shapes follow the layer sizes the pages describe: Switch-Base
(d_model 768, d_ff 3072) and Switch-Large (1024 / 4096), and one GPU's share
of the 2048-expert Switch-C model (kasblo explainer "Switch Transformerとは？",
section 論文の「高速化」をどう読むか).  The weight scale follows the paper's
reduced initialization, scale 0.1 instead of 1.0 (llm-papers-study close
reading "精读 06 | Switch Transformers", section 3.5, trick 2): truncated
normal with std sqrt(0.1 / fan_in), truncated at two standard deviations.
Hidden states stand in as x ~ N(0, 1) since no dataset is involved.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

TENSOR_X, TENSOR_WR, TENSOR_WIN, TENSOR_WOUT = 0, 1, 2, 3
ALPHA = 0.01


@dataclass(frozen=True)
class Spec:
    """One synthetic layer workload (shapes, dtypes, seed)."""
    name: str
    T: int
    d: int
    F: int
    N: int
    c: float
    act: str = "bf16"        # dtype of x / out / expert activations: "f32" | "bf16"
    expert: str = "bf16"     # dtype of W_in / W_out: "f32" | "bf16"
    seed: int = 0
    zipf: Optional[tuple] = None   # (s, beta): router bias b_i = beta * ln(Zipf_s(i))
    alpha: float = ALPHA
    capacity_override: int = 0

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


CONFIGS = {
    1: Spec("tiny-fp32", T=64, d=32, F=64, N=4, c=1.25, act="f32", expert="f32", seed=1),
    2: Spec("switch-base-8e", T=4096, d=768, F=3072, N=8, c=1.25, seed=2),
    3: Spec("zipf-overflow-128e", T=16384, d=768, F=3072, N=128, c=1.0, seed=3, zipf=(1.1, 0.12)),
    4: Spec("switch-large-128e", T=32768, d=1024, F=4096, N=128, c=1.25, seed=4),
    5: Spec("switch-c-share-2048e", T=131072, d=2048, F=6144, N=2048, c=1.0, seed=5),
}

# (tensor id, truncated, std as a function of the spec)
def tensor_law(spec: Spec, tensor_id: int):
    if tensor_id == TENSOR_X:
        return False, 1.0
    if tensor_id in (TENSOR_WR, TENSOR_WIN):
        return True, math.sqrt(0.1 / spec.d)
    if tensor_id == TENSOR_WOUT:
        return True, math.sqrt(0.1 / spec.F)
    raise ValueError(tensor_id)


_host = None
_gpu = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        for name, ptr in (("synth_fill_f32", ctypes.c_void_p), ("synth_fill_bf16", ctypes.c_void_p)):
            f = getattr(lib, name)
            f.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_double,
                          ctypes.c_uint64, ctypes.c_uint64, ptr, ctypes.c_int]
            f.restype = None
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_uint64]
        lib.synth_normal.restype = ctypes.c_double
        lib.synth_ln_export.argtypes = [ctypes.c_double]
        lib.synth_ln_export.restype = ctypes.c_double
        _host = lib
    return _host


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def fill(seed: int, tensor_id: int, truncated: bool, std: float, start: int, count: int,
         dtype: str, nthreads: int = 0) -> np.ndarray:
    """Elements [start, start+count) of one tensor: float32, or bf16 bit patterns as uint16."""
    lib = _load_host()
    nt = nthreads or host_threads()
    if dtype == "f32":
        out = np.empty(count, dtype=np.float32)
        lib.synth_fill_f32(seed, tensor_id, int(truncated), std, start, count,
                           out.ctypes.data_as(ctypes.c_void_p), nt)
    elif dtype == "bf16":
        out = np.empty(count, dtype=np.uint16)
        lib.synth_fill_bf16(seed, tensor_id, int(truncated), std, start, count,
                            out.ctypes.data_as(ctypes.c_void_p), nt)
    else:
        raise ValueError(dtype)
    return out


def normal(seed: int, tensor_id: int, truncated: bool, index: int) -> float:
    return _load_host().synth_normal(seed, tensor_id, int(truncated), index)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(a) if dtype == "bf16" else a


def router_bias(spec: Spec) -> Optional[np.ndarray]:
    """Per-expert router bias whose softmax mass follows Zipf(s): expert i has rank i+1."""
    if spec.zipf is None:
        return None
    s, beta = spec.zipf
    ranks = np.arange(1, spec.N + 1, dtype=np.float64)
    w = ranks ** (-s)
    p = w / w.sum()
    return (beta * np.log(p)).astype(np.float32)


def tensor(spec: Spec, tensor_id: int, start: int = 0, count: Optional[int] = None,
           nthreads: int = 0) -> np.ndarray:
    """Host copy of (a slice of) one input tensor, flattened, in its storage dtype."""
    shape = tensor_shape(spec, tensor_id)
    total = int(np.prod(shape))
    if count is None:
        count = total - start
    truncated, std = tensor_law(spec, tensor_id)
    dt = tensor_dtype(spec, tensor_id)
    return fill(spec.seed, tensor_id, truncated, std, start, count, dt, nthreads)


def tensor_shape(spec: Spec, tensor_id: int):
    return {TENSOR_X: (spec.T, spec.d), TENSOR_WR: (spec.N, spec.d),
            TENSOR_WIN: (spec.N, spec.F, spec.d), TENSOR_WOUT: (spec.N, spec.d, spec.F)}[tensor_id]


def tensor_dtype(spec: Spec, tensor_id: int) -> str:
    if tensor_id == TENSOR_X:
        return spec.act
    if tensor_id == TENSOR_WR:
        return "f32"
    return spec.expert


def host_inputs(spec: Spec, with_experts: bool = True, nthreads: int = 0) -> dict:
    """All inputs of a workload as host arrays in storage dtype (uint16 = bf16 bits)."""
    out = {
        "x": tensor(spec, TENSOR_X, nthreads=nthreads).reshape(spec.T, spec.d),
        "W_r": tensor(spec, TENSOR_WR, nthreads=nthreads).reshape(spec.N, spec.d),
        "b_r": router_bias(spec),
    }
    if with_experts:
        out["W_in"] = tensor(spec, TENSOR_WIN, nthreads=nthreads).reshape(spec.N, spec.F, spec.d)
        out["W_out"] = tensor(spec, TENSOR_WOUT, nthreads=nthreads).reshape(spec.N, spec.d, spec.F)
    return out


def expert_slice(spec: Spec, tensor_id: int, e: int, nthreads: int = 0) -> np.ndarray:
    """One expert's W_in [F,d] or W_out [d,F], regenerated on the host."""
    per = spec.F * spec.d
    a = tensor(spec, tensor_id, start=e * per, count=per, nthreads=nthreads)
    return a.reshape((spec.F, spec.d) if tensor_id == TENSOR_WIN else (spec.d, spec.F))


# ---------------------------------------------------------------- device side

def _load_gpu():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        lib.synth_gpu_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_double,
                                       ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_gpu_fill.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def gpu_fill(spec: Spec, tensor_id: int, dev_ptr: int, start: int, count: int, stream: int = 0):
    """Write elements [start, start+count) of a tensor straight into device memory."""
    truncated, std = tensor_law(spec, tensor_id)
    dt = tensor_dtype(spec, tensor_id)
    rc = _load_gpu().synth_gpu_fill(spec.seed, tensor_id, int(truncated), std, start, count,
                                    int(dt == "bf16"), ctypes.c_void_p(dev_ptr), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill failed: hipError {rc}")
