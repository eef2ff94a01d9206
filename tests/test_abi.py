"""The C ABI: the library loads, exports what include/*.h declares, and rejects
bad arguments before touching the GPU (host-side checks only, no compute)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(switch_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("switch_layer_create", "switch_route", "switch_forward", "switch_layer_destroy",
                 "switch_workspace_bytes", "switch_route_from_logits", "switch_forward_debug"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from switch_transformer_top_amd import binding as B
    for name in _declared_functions():
        assert hasattr(B.lib, name), f"{name} not exported"
        assert name in B.EXPORTS


def test_null_and_invalid_arguments_are_rejected_without_a_gpu():
    from switch_transformer_top_amd import binding as B
    ok = dict(t_max=64, d_model=128, d_ff=256, n_experts=4, capacity_factor=1.0,
              capacity_override=0, alpha=0.01, act_dtype=B.SWITCH_BF16, expert_dtype=B.SWITCH_BF16)
    fake = 0x10000  # never dereferenced: every call below fails validation first
    h = ctypes.c_void_p()

    def create(**kw):
        cfg = B.switch_config(**{**ok, **kw})
        return B.lib.switch_layer_create(ctypes.byref(cfg), fake, None, fake, fake, ctypes.byref(h))

    assert create(n_experts=0) == B.SWITCH_E_INVALID
    assert create(n_experts=9000) == B.SWITCH_E_INVALID
    assert create(d_model=100) == B.SWITCH_E_INVALID
    assert create(d_ff=0) == B.SWITCH_E_INVALID
    assert create(capacity_factor=-1.0) == B.SWITCH_E_INVALID
    assert create(capacity_factor=float("nan")) == B.SWITCH_E_INVALID
    assert create(t_max=-1) == B.SWITCH_E_INVALID
    assert create(act_dtype=7) == B.SWITCH_E_INVALID
    assert create(expert_dtype=B.SWITCH_F32) == B.SWITCH_E_UNSUPPORTED
    assert create(d_model=136) == B.SWITCH_E_UNSUPPORTED        # bf16 tiles need multiples of 128
    assert create(top_k=3) == B.SWITCH_E_INVALID                 # one or two experts per token
    assert create(top_k=-1) == B.SWITCH_E_INVALID
    assert create(top_k=2, n_experts=1) == B.SWITCH_E_INVALID    # k <= N
    cfg = B.switch_config(**ok)
    assert B.lib.switch_layer_create(ctypes.byref(cfg), None, None, fake, fake,
                                     ctypes.byref(h)) == B.SWITCH_E_INVALID
    assert B.lib.switch_layer_create(ctypes.byref(cfg), fake + 4, None, fake, fake,
                                     ctypes.byref(h)) == B.SWITCH_E_INVALID   # misaligned
    assert B.lib.switch_layer_create(None, fake, None, fake, fake, ctypes.byref(h)) == B.SWITCH_E_INVALID
    # calls on a NULL handle
    assert B.switch_workspace_bytes(None, 10) == 0
    assert B.switch_capacity(None, 10) == -1
    assert B.switch_forward(None, fake, 1, fake, fake, fake, fake, fake, fake, None, None, fake,
                            1 << 20) == B.SWITCH_E_INVALID
    assert B.switch_route(None, fake, 1, None, fake, fake, fake, fake, fake, None, fake,
                          1 << 20) == B.SWITCH_E_INVALID
    assert B.lib.switch_profile_read(None, None, None, 4) == -1
    B.switch_layer_destroy(None)


def test_status_strings():
    from switch_transformer_top_amd import binding as B
    for s in (0, 1, 2, 3):
        assert B.status_string(s).startswith("SWITCH_")
    assert "unknown" in B.status_string(99)


def test_product_path_does_not_touch_the_oracle():
    """The library and binding never reference the oracle or its library."""
    srcs = glob.glob(os.path.join(ROOT, "switch_transformer_top_amd", "**", "*.*"), recursive=True)
    for p in srcs:
        if p.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
            text = open(p, encoding="utf-8").read()
            assert "oracle" not in text.lower(), p
