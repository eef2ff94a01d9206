"""switch_forward_noalloc (the forward for callers that cannot allocate device
memory) against switch_forward, through the C ABI: the same kernels on the
library's fixed scratch array instead of a caller workspace must give the same
bits, on two calls in a row with the second one smaller, and a call that needs
more than the array must be refused before anything is launched."""
import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

OUTS = ("out", "expert_idx", "gate", "position", "drop_mask", "aux_loss", "logits", "load")


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from switch_transformer_top_amd import binding
    return binding


def _reference(B, layer, x, T, stream):
    b = layer.alloc(T)
    layer.forward(x, T, b, stream=stream, with_logits=True)
    return b


def _noalloc(B, layer, x, T, stream):
    b = layer.alloc(T)   # outputs only; the call takes no workspace
    for v in b.values():
        if hasattr(v, "fill_") and v is not b["ws"]:
            v.fill_(0)   # stale values must not survive the call
    st = B.switch_forward_noalloc(layer.handle, x, T, b["out"], b["expert_idx"], b["gate"],
                                  b["position"], b["drop_mask"], b["aux_loss"], b["logits"],
                                  b["load"], stream)
    assert st == B.SWITCH_OK, B.status_string(st)
    return b


def _same(ref, got, tag):
    torch.cuda.synchronize()
    for k in OUTS:
        a = _host(ref[k])
        g = _host(got[k])
        assert a.shape == g.shape, (tag, k)
        assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"{tag}: {k} differs"


def _host(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("shape", [
    dict(T=2000, N=8, d=256, F=512, seed=31),       # token-chunk router, one-launch assignment
    dict(T=1500, N=300, d=128, F=256, seed=32),     # logits router, scan + slot kernel
])
def test_noalloc_matches_forward_twice_second_smaller(B, shape):
    spec = S.CONFIGS[2].with_(**shape)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    stream = torch.cuda.current_stream().cuda_stream
    x = B.to_device(host["x"], torch.device("cuda:0"))
    for T in (spec.T, spec.T // 3 + 1):
        print(f"[case] noalloc {spec.name} T={T} N={spec.N} d={spec.d} F={spec.F}", flush=True)
        assert B.switch_workspace_bytes(layer.handle, T) <= B.SWITCH_NOALLOC_SCRATCH_BYTES
        got = _noalloc(B, layer, x, T, stream)
        ref = _reference(B, layer, x, T, stream)
        _same(ref, got, f"T={T}")


def test_noalloc_switch_base_shape_and_refusal(B):
    """The Switch-Base workload fits the array; twice its tokens do not, and that call
    returns SWITCH_E_TOO_LARGE without writing any output."""
    spec = S.CONFIGS[2]
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, t_max=2 * spec.T)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    print(f"[case] noalloc {spec.name} T={spec.T}", flush=True)
    x = B.to_device(host["x"], dev)
    got = _noalloc(B, layer, x, spec.T, stream)
    ref = _reference(B, layer, x, spec.T, stream)
    _same(ref, got, spec.name)

    T2 = 2 * spec.T
    assert B.switch_workspace_bytes(layer.handle, T2) > B.SWITCH_NOALLOC_SCRATCH_BYTES
    x2 = torch.cat([x, x])
    b = layer.alloc(T2)
    b["out"].fill_(7)
    b["expert_idx"].fill_(-5)
    print(f"[case] noalloc refusal T={T2}", flush=True)
    st = B.switch_forward_noalloc(layer.handle, x2, T2, b["out"], b["expert_idx"], b["gate"],
                                  b["position"], b["drop_mask"], b["aux_loss"], b["logits"],
                                  b["load"], stream)
    assert st == B.SWITCH_E_TOO_LARGE
    assert "no-allocation" in B.status_string(st)
    torch.cuda.synchronize()
    assert bool((b["out"] == 7).all()) and bool((b["expert_idx"] == -5).all())
    # the layer still works on the array after the refusal
    got = _noalloc(B, layer, x, spec.T // 2, stream)
    ref = _reference(B, layer, x, spec.T // 2, stream)
    _same(ref, got, "after refusal")


def test_noalloc_rejects_bad_arguments_before_launch(B):
    spec = S.CONFIGS[2].with_(T=256, N=8, d=128, F=256, seed=33)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    assert B.switch_forward_noalloc(None, 0, 1, 0, 0, 0, 0, 0, 0, None, None) == B.SWITCH_E_INVALID
    b = layer.alloc(spec.T)
    x = B.to_device(host["x"], torch.device("cuda:0"))
    # T above t_max, then a NULL required output
    assert B.switch_forward_noalloc(layer.handle, x, spec.T + 1, b["out"], b["expert_idx"],
                                    b["gate"], b["position"], b["drop_mask"], b["aux_loss"],
                                    None, None) == B.SWITCH_E_INVALID
    assert B.switch_forward_noalloc(layer.handle, x, spec.T, None, b["expert_idx"], b["gate"],
                                    b["position"], b["drop_mask"], b["aux_loss"], None,
                                    None) == B.SWITCH_E_INVALID
