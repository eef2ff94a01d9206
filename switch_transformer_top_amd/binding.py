"""ctypes binding of libswitch_layer.so (include/switch_layer.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  The functions keep the C names; tensors may be passed as torch
CUDA tensors (their data_ptr is taken) or as raw integer device addresses.
There is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libswitch_layer.so")

SWITCH_OK, SWITCH_E_INVALID, SWITCH_E_UNSUPPORTED, SWITCH_E_HIP = 0, 1, 2, 3
SWITCH_E_TOO_LARGE = 4
SWITCH_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/switch_layer.h
SWITCH_F32, SWITCH_BF16 = 0, 1
SWITCH_FFN_AUTO, SWITCH_FFN_UNFUSED, SWITCH_FFN_FUSED = 0, 1, 2

EXPORTS = ("switch_layer_create", "switch_layer_destroy", "switch_capacity",
           "switch_workspace_bytes", "switch_route", "switch_forward",
           "switch_route_from_logits", "switch_forward_debug", "switch_profile_enable",
           "switch_profile_read", "switch_status_string", "switch_last_async_error",
           "switch_backward", "switch_backward_workspace_bytes", "switch_set_keep_expert_out",
           "switch_forward_noalloc", "switch_set_ffn_mode")


class switch_config(ctypes.Structure):
    _fields_ = [("t_max", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("capacity_factor", ctypes.c_double),
                ("capacity_override", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32),
                ("top_k", ctypes.c_int32)]


class SwitchError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
lib.switch_layer_create.argtypes = [ctypes.POINTER(switch_config), _vp, _vp, _vp, _vp,
                                    ctypes.POINTER(_vp)]
lib.switch_layer_create.restype = ctypes.c_int
lib.switch_layer_destroy.argtypes = [_vp]
lib.switch_layer_destroy.restype = None
lib.switch_capacity.argtypes = [_vp, _i64]
lib.switch_capacity.restype = _i64
lib.switch_workspace_bytes.argtypes = [_vp, _i64]
lib.switch_workspace_bytes.restype = _sz
lib.switch_route.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.switch_route.restype = ctypes.c_int
lib.switch_forward.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                               _vp]
lib.switch_forward.restype = ctypes.c_int
lib.switch_forward_noalloc.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp]
lib.switch_forward_noalloc.restype = ctypes.c_int
lib.switch_route_from_logits.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                         _vp]
lib.switch_route_from_logits.restype = ctypes.c_int
lib.switch_forward_debug.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _sz, _vp, _vp]
lib.switch_forward_debug.restype = ctypes.c_int
lib.switch_backward.argtypes = [_vp, _vp, _i64, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]
lib.switch_backward.restype = ctypes.c_int
lib.switch_backward_workspace_bytes.argtypes = [_vp, _i64]
lib.switch_backward_workspace_bytes.restype = _sz
lib.switch_profile_enable.argtypes = [_vp, ctypes.c_int]
lib.switch_profile_enable.restype = ctypes.c_int
lib.switch_set_ffn_mode.argtypes = [_vp, ctypes.c_int]
lib.switch_set_ffn_mode.restype = ctypes.c_int
lib.switch_set_keep_expert_out.argtypes = [_vp, ctypes.c_int]
lib.switch_set_keep_expert_out.restype = ctypes.c_int
lib.switch_profile_read.argtypes = [_vp, ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(ctypes.c_char_p), ctypes.c_int]
lib.switch_profile_read.restype = ctypes.c_int
lib.switch_status_string.argtypes = [ctypes.c_int]
lib.switch_status_string.restype = ctypes.c_char_p
lib.switch_last_async_error.argtypes = [_vp, _vp]
lib.switch_last_async_error.restype = ctypes.c_int


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def status_string(status: int) -> str:
    return lib.switch_status_string(status).decode()


def _check(status: int, what: str):
    if status != SWITCH_OK:
        raise SwitchError(status, what)


# ------------------------------------------------------------------ C-named calls

def switch_layer_create(cfg: switch_config, W_r, b_r, W_in, W_out) -> int:
    h = _vp()
    _check(lib.switch_layer_create(ctypes.byref(cfg), _ptr(W_r), _ptr(b_r), _ptr(W_in),
                                   _ptr(W_out), ctypes.byref(h)), "switch_layer_create")
    return h.value


def switch_layer_destroy(handle: int) -> None:
    lib.switch_layer_destroy(handle)


def switch_capacity(handle: int, T: int) -> int:
    return lib.switch_capacity(handle, T)


def switch_workspace_bytes(handle: int, T: int) -> int:
    return lib.switch_workspace_bytes(handle, T)


def switch_route(handle, x, T, logits, expert_idx, gate, position, drop_mask, aux_loss, load, ws,
                 ws_bytes, stream=0) -> int:
    return lib.switch_route(handle, _ptr(x), T, _ptr(logits), _ptr(expert_idx), _ptr(gate),
                            _ptr(position), _ptr(drop_mask), _ptr(aux_loss), _ptr(load), _ptr(ws),
                            ws_bytes, stream)


def switch_forward(handle, x, T, out, expert_idx, gate, position, drop_mask, aux_loss, logits,
                   load, ws, ws_bytes, stream=0) -> int:
    return lib.switch_forward(handle, _ptr(x), T, _ptr(out), _ptr(expert_idx), _ptr(gate),
                              _ptr(position), _ptr(drop_mask), _ptr(aux_loss), _ptr(logits),
                              _ptr(load), _ptr(ws), ws_bytes, stream)


def switch_forward_noalloc(handle, x, T, out, expert_idx, gate, position, drop_mask, aux_loss,
                           logits, load, stream=0) -> int:
    return lib.switch_forward_noalloc(handle, _ptr(x), T, _ptr(out), _ptr(expert_idx), _ptr(gate),
                                      _ptr(position), _ptr(drop_mask), _ptr(aux_loss),
                                      _ptr(logits), _ptr(load), stream)


def switch_route_from_logits(handle, logits, T, expert_idx, gate, position, drop_mask, aux_loss,
                             load, ws, ws_bytes, stream=0) -> int:
    return lib.switch_route_from_logits(handle, _ptr(logits), T, _ptr(expert_idx), _ptr(gate),
                                        _ptr(position), _ptr(drop_mask), _ptr(aux_loss),
                                        _ptr(load), _ptr(ws), ws_bytes, stream)


def switch_forward_debug(handle, x, T, out, expert_idx, gate, position, drop_mask, aux_loss,
                         logits, load, ws, ws_bytes, expert_out, stream=0) -> int:
    return lib.switch_forward_debug(handle, _ptr(x), T, _ptr(out), _ptr(expert_idx), _ptr(gate),
                                    _ptr(position), _ptr(drop_mask), _ptr(aux_loss),
                                    _ptr(logits), _ptr(load), _ptr(ws), ws_bytes,
                                    _ptr(expert_out), stream)


def switch_backward(handle, x, T, grad_out, grad_aux, logits, expert_idx, gate, position,
                    drop_mask, load, grad_x, grad_W_r, grad_b_r, grad_W_in, grad_W_out, ws,
                    ws_bytes, fwd_ws=None, fwd_ws_bytes=0, stream=0) -> int:
    return lib.switch_backward(handle, _ptr(x), T, _ptr(grad_out), float(grad_aux), _ptr(logits),
                               _ptr(expert_idx), _ptr(gate), _ptr(position), _ptr(drop_mask),
                               _ptr(load), _ptr(grad_x), _ptr(grad_W_r), _ptr(grad_b_r),
                               _ptr(grad_W_in), _ptr(grad_W_out), _ptr(ws), ws_bytes,
                               _ptr(fwd_ws), fwd_ws_bytes, stream)


def switch_backward_workspace_bytes(handle: int, T: int) -> int:
    return lib.switch_backward_workspace_bytes(handle, T)


def switch_set_keep_expert_out(handle: int, keep: bool) -> None:
    """Training forward: later forward calls also store the expert outputs in their
    workspace, for a backward given that workspace."""
    _check(lib.switch_set_keep_expert_out(handle, 1 if keep else 0), "switch_set_keep_expert_out")


def switch_set_ffn_mode(handle: int, mode: int) -> None:
    """Expert FFN variant of later forward calls: SWITCH_FFN_AUTO, _UNFUSED or _FUSED."""
    _check(lib.switch_set_ffn_mode(handle, int(mode)), "switch_set_ffn_mode")


def switch_profile_enable(handle: int, max_calls: int) -> None:
    _check(lib.switch_profile_enable(handle, int(max_calls)), "switch_profile_enable")


def switch_profile_read(handle: int, cap: int = 24):
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    n = lib.switch_profile_read(handle, ms, names, cap)
    if n < 0:
        raise SwitchError(SWITCH_E_HIP, "switch_profile_read")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


def switch_last_async_error(handle, stream=0) -> int:
    return lib.switch_last_async_error(handle, stream)


# ------------------------------------------------------------------ convenience wrapper

class SwitchLayer:
    """Owns a handle, its device weights (torch tensors) and device output buffers.

    Only allocation and argument passing happen here; all compute is the library's.
    """

    def __init__(self, cfg: switch_config, W_r, b_r, W_in, W_out):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.weights = (W_r, b_r, W_in, W_out)   # kept alive: the library borrows them
        self.device = W_r.device
        self.handle = switch_layer_create(cfg, W_r, b_r, W_in, W_out)
        self._ws = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                switch_layer_destroy(h)
            except TypeError:   # interpreter shutdown: the module is already torn down
                pass
            self.handle = None

    # -- construction from the synthetic generator's host arrays
    @classmethod
    def from_host(cls, spec, host: dict, device=None, t_max: Optional[int] = None,
                  top_k: int = 1):
        import torch
        dev = device or torch.device("cuda:0")
        act = SWITCH_BF16 if spec.act == "bf16" else SWITCH_F32
        exp = SWITCH_BF16 if spec.expert == "bf16" else SWITCH_F32
        cfg = switch_config(t_max=t_max if t_max is not None else spec.T, d_model=spec.d,
                            d_ff=spec.F, n_experts=spec.N, capacity_factor=spec.c,
                            capacity_override=spec.capacity_override, alpha=spec.alpha,
                            act_dtype=act, expert_dtype=exp, top_k=top_k)
        W_r = torch.from_numpy(np.ascontiguousarray(host["W_r"])).to(dev)
        b_r = None if host.get("b_r") is None else torch.from_numpy(host["b_r"]).to(dev)
        W_in = to_device(host["W_in"], dev)
        W_out = to_device(host["W_out"], dev)
        return cls(cfg, W_r, b_r, W_in, W_out)

    def alloc(self, T: int) -> dict:
        torch = self.torch
        dev = self.device
        es = 2 if self.cfg.act_dtype == SWITCH_BF16 else 4
        N, d = self.cfg.n_experts, self.cfg.d_model
        nbytes = switch_workspace_bytes(self.handle, T)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        xdt = torch.int16 if es == 2 else torch.float32
        k = max(1, int(self.cfg.top_k))
        per = (T,) if k == 1 else (T, k)   # per-token outputs: [T] for top-1, [T, k] otherwise
        return dict(
            out=torch.empty((T, d), dtype=xdt, device=dev),
            expert_idx=torch.empty(per, dtype=torch.int32, device=dev),
            gate=torch.empty(per, dtype=torch.float32, device=dev),
            position=torch.empty(per, dtype=torch.int32, device=dev),
            drop_mask=torch.empty(per, dtype=torch.uint8, device=dev),
            aux_loss=torch.empty(1, dtype=torch.float32, device=dev),
            logits=torch.empty((T, N), dtype=torch.float32, device=dev),
            load=torch.empty(N, dtype=torch.int32, device=dev),
            ws=self._ws, ws_bytes=nbytes)

    def forward(self, x, T: int, bufs: dict, stream: int = 0, with_logits: bool = True,
                expert_out=None):
        b = bufs
        args = (self.handle, x, T, b["out"], b["expert_idx"], b["gate"], b["position"],
                b["drop_mask"], b["aux_loss"], b["logits"] if with_logits else None, b["load"],
                b["ws"], b["ws_bytes"])
        if expert_out is None:
            st = switch_forward(*args, stream)
        else:
            st = switch_forward_debug(*args, expert_out, stream)
        _check(st, "switch_forward")

    def route(self, x, T: int, bufs: dict, stream: int = 0):
        b = bufs
        _check(switch_route(self.handle, x, T, b["logits"], b["expert_idx"], b["gate"],
                            b["position"], b["drop_mask"], b["aux_loss"], b["load"], b["ws"],
                            b["ws_bytes"], stream), "switch_route")

    def route_from_logits(self, logits, T: int, bufs: dict, stream: int = 0):
        b = bufs
        _check(switch_route_from_logits(self.handle, logits, T, b["expert_idx"], b["gate"],
                                        b["position"], b["drop_mask"], b["aux_loss"], b["load"],
                                        b["ws"], b["ws_bytes"], stream), "switch_route_from_logits")

    def alloc_backward(self, T: int) -> dict:
        """Gradient outputs and the backward workspace (device tensors)."""
        torch = self.torch
        dev = self.device
        N, d, F = self.cfg.n_experts, self.cfg.d_model, self.cfg.d_ff
        nbytes = switch_backward_workspace_bytes(self.handle, T)
        return dict(
            grad_x=torch.empty((T, d), dtype=torch.int16, device=dev),
            grad_W_r=torch.empty((N, d), dtype=torch.float32, device=dev),
            grad_b_r=torch.empty(N, dtype=torch.float32, device=dev),
            grad_W_in=torch.empty((N, F, d), dtype=torch.int16, device=dev),
            grad_W_out=torch.empty((N, d, F), dtype=torch.int16, device=dev),
            ws=torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev), ws_bytes=nbytes)

    def backward(self, x, T: int, grad_out, grad_aux: float, fwd: dict, grads: dict,
                 stream: int = 0, reuse_forward: bool = False):
        """Gradients at the routing of a forward call whose outputs are in fwd (logits
        included).  With reuse_forward the forward's workspace (fwd["ws"]) supplies the
        expert activations H instead of a recomputation: every alloc() of a layer shares
        that workspace, so no other forward or routing call of the layer may run between
        the two."""
        g = grads
        fws = fwd["ws"] if reuse_forward else None
        fwb = fwd["ws_bytes"] if reuse_forward else 0
        _check(switch_backward(self.handle, x, T, grad_out, grad_aux, fwd["logits"],
                               fwd["expert_idx"], fwd["gate"], fwd["position"], fwd["drop_mask"],
                               fwd["load"], g["grad_x"], g["grad_W_r"], g["grad_b_r"],
                               g["grad_W_in"], g["grad_W_out"], g["ws"], g["ws_bytes"], fws, fwb,
                               stream),
               "switch_backward")

    def forward_host(self, x_host: np.ndarray, debug: bool = False) -> dict:
        """Upload x, run the layer on the current stream, download every output."""
        torch = self.torch
        T = x_host.shape[0]
        x = to_device(x_host, self.device)
        b = self.alloc(T)
        eo = None
        if debug:
            Cb = max(0, min(switch_capacity(self.handle, T), T))
            es_dt = torch.int16 if self.cfg.act_dtype == SWITCH_BF16 else torch.float32
            eo = torch.zeros((self.cfg.n_experts, Cb, self.cfg.d_model), dtype=es_dt,
                             device=self.device)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        self.forward(x, T, b, stream=stream, expert_out=eo)
        torch.cuda.synchronize(self.device)
        res = {k: from_device(v) for k, v in b.items() if k not in ("ws", "ws_bytes")}
        res["aux_loss"] = float(res["aux_loss"][0])
        if eo is not None:
            res["expert_out"] = from_device(eo)
        return res


def to_device(a: np.ndarray, dev):
    """Host array (uint16 = bf16 bits, or float32/int) -> torch device tensor, same bytes."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev)
    return torch.from_numpy(a).to(dev)


def from_device(t) -> np.ndarray:
    import torch
    a = t.detach().cpu().numpy()
    if t.dtype == torch.int16:
        return a.view(np.uint16)
    return a
