"""No kernel writes past the end of an output or of the workspace.

Each forward below takes a different set of kernels: the small-N router, the
token-split router and the logits router; the one-launch and the two-launch
capacity assignment; 256 x 256 tiles (gathered rows, the fused combine),
split-K 128 x 128 tiles, 128- and 64-row tiles with more tiles than CUs; top-1
and top-2.  Every output and the workspace is a view into a larger buffer whose
tail holds a fill pattern that must survive the call; the results are also
checked against the oracle's routing."""
import numpy as np
import pytest

import oracle
import synthetic as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GUARD = 4096  # bytes of fill after every buffer


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from switch_transformer_top_amd import binding
    return binding


def _guarded(t, fill):
    """A tensor shaped like t, followed in memory by at least GUARD bytes of fill."""
    n = t.numel()
    extra = (GUARD + t.element_size() - 1) // t.element_size()
    big = torch.full((n + extra,), fill, dtype=t.dtype, device=t.device)
    return big, big[:n].view(t.shape)


@pytest.mark.parametrize("T,N,d,F,c,k,seed", [
    (4096, 8, 768, 3072, 1.25, 1, 111),     # Switch-Base: wide GEMM1, split-K GEMM2 + combine
    (2100, 4, 256, 768, 1.0, 1, 112),       # ragged tiles and drops, split-K for both matmuls
    (9600, 32, 1024, 256, 1.0, 1, 113),     # token-split router, wide GEMM2 + combine
    (8192, 256, 256, 256, 1.0, 1, 114),     # two-launch assignment, 64-row tiles
    (12000, 128, 128, 512, 1.25, 1, 115),   # 128-row tiles with more tiles than CUs
    (600, 300, 128, 128, 1.0, 1, 116),      # logits router (N > 256)
    (1000, 520, 128, 256, 1.0, 1, 118),     # logits router, partial expert tile and token group
    (4096, 8, 768, 3072, 1.25, 2, 117),     # top-2: wide GEMM1, 128-row GEMM2, the combine pass
])
def test_no_writes_past_the_end(B, T, N, d, F, c, k, seed):
    spec = S.Spec(f"guard-{T}-{N}-k{k}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, top_k=k)
    print(f"[case] {spec.name}", flush=True)
    x = B.to_device(host["x"], layer.device)
    bufs = layer.alloc(T)
    fills = {"out": 0x3C3C, "expert_idx": -7, "gate": -1.5, "position": -12345,
             "drop_mask": 0xA5, "aux_loss": -2.5, "logits": 7.25, "load": -3}
    bigs = {}
    for key, fill in fills.items():
        bigs[key], bufs[key] = _guarded(bufs[key], fill)
    ws_big = torch.full((bufs["ws_bytes"] + GUARD,), 0x5A, dtype=torch.uint8, device=layer.device)
    bufs["ws"] = ws_big[:bufs["ws_bytes"]]
    layer.forward(x, T, bufs)
    torch.cuda.synchronize()
    for key, fill in fills.items():
        big = bigs[key]
        tail = B.from_device(big[bufs[key].numel():])
        want = np.asarray(fill).astype(tail.dtype)
        assert np.all(tail == want), f"{spec.name}: {key} written past its end"
    ws_tail = B.from_device(ws_big[bufs["ws_bytes"]:])
    assert np.all(ws_tail == 0x5A), f"{spec.name}: workspace written past its end"
    # and the routing is still the oracle's on the GPU's logits
    h = B.from_device(bufs["logits"]).astype(np.float64)
    ref = oracle.route(h, c) if k == 1 else oracle.route_topk(h, k, c)
    assert np.array_equal(B.from_device(bufs["expert_idx"]), ref["expert_idx"])
    assert np.array_equal(B.from_device(bufs["position"]), ref["position"])
    assert np.array_equal(B.from_device(bufs["drop_mask"]), ref["drop"])


@pytest.mark.parametrize("T,N,d,F,c,k,seed", [
    (4096, 8, 768, 3072, 1.25, 1, 121),     # Switch-Base: 256 x 256 and split-K products
    (777, 5, 128, 384, 1.25, 1, 122),       # odd expert count, ragged K of the weight gradients
    (600, 300, 128, 128, 1.0, 1, 123),      # N > 256: logits router, many small experts
    (1000, 8, 256, 512, 1.0, 2, 124),       # top-2
])
def test_backward_no_writes_past_the_end(B, T, N, d, F, c, k, seed):
    spec = S.Spec(f"guard-bwd-{T}-{N}-k{k}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, top_k=k)
    print(f"[case] {spec.name}", flush=True)
    x = B.to_device(host["x"], layer.device)
    fwd = layer.alloc(T)
    layer.forward(x, T, fwd)
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((T, d)).astype(np.float32)
    G = B.to_device((g.view(np.uint32) >> 16).astype(np.uint16), layer.device)  # truncated to bf16
    grads = layer.alloc_backward(T)
    fills = {"grad_x": 0x3C3C, "grad_W_r": -1.25, "grad_b_r": -2.5, "grad_W_in": 0x3C3C,
             "grad_W_out": 0x3C3C}
    bigs = {}
    for key, fill in fills.items():
        bigs[key], grads[key] = _guarded(grads[key], fill)
    ws_big = torch.full((grads["ws_bytes"] + GUARD,), 0x5A, dtype=torch.uint8,
                        device=layer.device)
    grads["ws"] = ws_big[:grads["ws_bytes"]]
    for reuse in (False, True):
        layer.backward(x, T, G, 1.0, fwd, grads, reuse_forward=reuse)
        torch.cuda.synchronize()
        for key, fill in fills.items():
            tail = B.from_device(bigs[key][grads[key].numel():])
            assert np.all(tail == np.asarray(fill).astype(tail.dtype)), \
                f"{spec.name}: {key} written past its end"
        assert np.all(B.from_device(ws_big[grads["ws_bytes"]:]) == 0x5A), \
            f"{spec.name}: backward workspace written past its end"
