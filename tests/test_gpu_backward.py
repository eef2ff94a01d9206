"""GPU parity of the backward pass (the next row after the forward) against the
oracle's backward, through the C ABI.

The oracle is fed the GPU forward's routing and fp32 logits, so both sides
differentiate at the same routing.  The GPU rounds to bf16 (u = 2^-8 relative)
what the forward rounds: the scaled output gradient S = gate G, the activation
H = relu(U), the expert output Y, the gradient dU and every bf16 output once;
sums run in fp32.  The bars are the error bounds of those roundings, element by
element, summed the way each gradient sums its terms (abs values, per expert):
  H             |H - A| <= u |A| + gamma_d |X| |W_in|^T (fp32 sum, then rounding)
  grad_W_out[e] = S^T H     |S|^T |H - A| + (u + gamma_n) |S|^T |A| + u |ref|
  grad_W_in[e]  = dU^T X    ((2u + gamma_d) |S| |W_out| + amb * |S W_out|)^T |X| + ...,
                            amb marking ReLU inputs within the fp32 dot-product error
                            bound of 0 (their derivative may go either way)
  router        dg_t = G_t . Y_t off by |G_t| . (|Y error| + gamma_d |Y|);
                dh = p (dp - p . dp) moves by p_i |[i = e] - p_e| of that, plus a
                1e-6 relative allowance for the fp32 softmax; grad_W_r and
                grad_b_r sum |dh errors| |x| (and 2 gamma_T of the fp32 sum)
  grad_x        the expert part |W_in|^T |dU error| + u |dX| + the router part
                |dh error| |W_r| + u |ref| for the final rounding; the router part's
                products take two bf16 pieces of W_r and of dh (hi + mid, the
                rest below u^2 of the value) and leave out mid * mid and the rests,
                at most 3.1 u^2 |W_r| |dh| per product, on top of the fp32 sum
"""
import numpy as np
import pytest

import oracle
import synthetic as S

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from switch_transformer_top_amd import binding
    return binding


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


U16 = 2.0 ** -8            # bf16 unit roundoff (8-bit significand)
U32 = 2.0 ** -24           # fp32 unit roundoff


def _gamma(n):
    return n * U32 / (1 - n * U32)


def _within(got, ref, bound, tag):
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), f"{tag}: {bad.sum()} of {bad.size} off, worst " \
        f"{(err / (bound + 1e-300)).max():.3g} x the bound"


def _bounds(spec, host, f, Gf, ref, g_aux):
    """Error bounds of the GPU gradients (see the module docstring).  Routing
    arrays are [T] (top-1) or [T, k]; each kept assignment (t, j) contributes
    like a kept token of the top-1 layer."""
    xf = S.to_f32(host["x"], spec.act).astype(np.float64)
    W_in = S.to_f32(host["W_in"], spec.expert).astype(np.float64)
    W_out = S.to_f32(host["W_out"], spec.expert).astype(np.float64)
    W_r = host["W_r"].astype(np.float64)
    T, d, N, F = spec.T, spec.d, spec.N, spec.F
    eidx = f["expert_idx"].reshape(T, -1)
    k = eidx.shape[1]
    ea = eidx.reshape(-1)                                  # per assignment a = t k + j
    gate = f["gate"].astype(np.float64).reshape(-1)
    kept = (f["drop_mask"].reshape(-1) == 0)
    tok = np.repeat(np.arange(T), k)
    b = dict(dW_out=np.zeros((N, d, F)), dW_in=np.zeros((N, F, d)), dx=np.zeros((T, d)))
    ddg = np.zeros(T * k)       # bound on the error of dg_a = G_t . Y_a
    dg_abs = np.zeros(T * k)    # bound on |dg_a|
    for e in range(N):
        rows = np.flatnonzero(kept & (ea == e))
        if rows.size == 0:
            continue
        t_r = tok[rows]                                    # distinct: one choice per expert
        X = xf[t_r]
        n = rows.size
        Sg = gate[rows, None] * Gf[t_r]
        U = X @ W_in[e].T
        A = np.maximum(U, 0)
        XW = np.abs(X) @ np.abs(W_in[e]).T             # |X| |W_in|^T: scale of U
        amb = np.abs(U) <= 2 * _gamma(d) * XW           # ReLU sign not settled in fp32
        Aerr = U16 * np.abs(A) + _gamma(d) * XW         # |H - A|: fp32 sum, bf16 rounding
        DA = Sg @ W_out[e]
        DAabs = np.abs(Sg) @ np.abs(W_out[e])
        AW = np.abs(A) @ np.abs(W_out[e]).T             # bounds |Y|
        Yerr = Aerr @ np.abs(W_out[e]).T + (U16 + _gamma(F)) * AW
        b["dW_out"][e] = (np.abs(Sg).T @ Aerr + (U16 + _gamma(n)) * (np.abs(Sg).T @ np.abs(A))
                          + U16 * np.abs(ref["dW_out"][e]))
        ddu = (2 * U16 + _gamma(d)) * DAabs + amb * np.abs(DA)
        b["dW_in"][e] = ((ddu.T @ np.abs(X)) + _gamma(n) * (DAabs.T @ np.abs(X))
                         + U16 * np.abs(ref["dW_in"][e]))
        dXe_abs = DAabs @ np.abs(W_in[e])
        b["dx"][t_r] += ddu @ np.abs(W_in[e]) + (U16 + _gamma(F)) * dXe_abs
        ddg[rows] = (np.abs(Gf[t_r]) * Yerr).sum(1) + _gamma(d) * (np.abs(Gf[t_r]) * AW).sum(1)
        dg_abs[rows] = (np.abs(Gf[t_r]) * AW).sum(1)
    h = f["logits"].astype(np.float64)
    p = np.exp(h - h.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    c = abs(g_aux) * spec.alpha * N * f["load"].astype(np.float64) / (k * T * T)
    dp_abs = np.zeros((T, N)) + c[None, :]
    ddh = np.zeros((T, N))
    for j in range(k):
        a = np.arange(T) * k + j
        kj = kept[a].astype(np.float64)
        onehot = np.zeros((T, N))
        onehot[np.arange(T), eidx[:, j]] = kj
        dp_abs += onehot * dg_abs[a][:, None]
        pe = p[np.arange(T), eidx[:, j]]
        ddh += p * np.abs(onehot - (pe * kj)[:, None]) * ddg[a][:, None]
    dh_abs = p * (dp_abs + (p * dp_abs).sum(1, keepdims=True))
    ddh += 1e-6 * dh_abs
    b["dW_r"] = ddh.T @ np.abs(xf) + 2 * _gamma(T) * (dh_abs.T @ np.abs(xf))
    b["db"] = ddh.sum(0) + 2 * _gamma(T) * dh_abs.sum(0)
    b["dx"] += ddh @ np.abs(W_r) + (3.2 * U16 ** 2 + 2 * _gamma(N)) * (dh_abs @ np.abs(W_r))
    b["dx"] += U16 * np.abs(ref["dx"]) + 4 * U32 * (np.abs(Gf) + b["dx"])
    return b


def _run(B, spec, g_aux=1.0, seed=0, top_k=1):
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, top_k=top_k)
    print(f"[case] backward {spec.name} T={spec.T} d={spec.d} F={spec.F} N={spec.N} c={spec.c}",
          flush=True)
    T, d = spec.T, spec.d
    x = B.to_device(host["x"], layer.device)
    fwd = layer.alloc(T)
    layer.forward(x, T, fwd)
    rng = np.random.default_rng(1000 + spec.seed + seed)
    G_bits = _bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    G = B.to_device(G_bits, layer.device)
    grads = layer.alloc_backward(T)
    layer.backward(x, T, G, g_aux, fwd, grads)
    torch.cuda.synchronize()
    f = {k: B.from_device(v) for k, v in fwd.items() if k not in ("ws", "ws_bytes", "out")}
    g = {k: B.from_device(v) for k, v in grads.items() if k not in ("ws", "ws_bytes")}
    return host, layer, x, G, fwd, grads, f, g, G_bits


def _check(spec, host, f, g, G_bits, g_aux, tag):
    xf = S.to_f32(host["x"], spec.act)
    W_in = S.to_f32(host["W_in"], spec.expert)
    W_out = S.to_f32(host["W_out"], spec.expert)
    Gf = S.to_f32(G_bits, "bf16").astype(np.float64)
    args = (xf, host["W_r"], W_in, W_out, f["logits"].astype(np.float64), f["expert_idx"],
            f["gate"].astype(np.float64), f["drop_mask"], f["load"], Gf, g_aux, spec.alpha)
    ref = oracle.backward(*args) if f["expert_idx"].ndim == 1 else oracle.backward_topk(*args)
    b = _bounds(spec, host, f, Gf, ref, g_aux)
    _within(S.to_f32(g["grad_W_out"], "bf16"), ref["dW_out"], b["dW_out"], f"{tag} grad_W_out")
    _within(S.to_f32(g["grad_W_in"], "bf16"), ref["dW_in"], b["dW_in"], f"{tag} grad_W_in")
    _within(g["grad_W_r"].astype(np.float64), ref["dW_r"], b["dW_r"], f"{tag} grad_W_r")
    _within(g["grad_b_r"].astype(np.float64), ref["db"], b["db"], f"{tag} grad_b_r")
    _within(S.to_f32(g["grad_x"], "bf16").astype(np.float64), ref["dx"], b["dx"],
            f"{tag} grad_x")
    return ref


@pytest.mark.parametrize("T,N,d,F,c,seed", [
    (1000, 8, 256, 512, 1.0, 71),      # several M tiles, drops
    (777, 5, 128, 384, 1.25, 72),      # odd expert count, ragged K of the weight gradients
    (130, 16, 128, 256, 0.5, 73),      # heavy overflow
    (9, 32, 128, 128, 2.0, 74),        # T < N: experts with no token get zero gradients
    (700, 48, 128, 256, 1.0, 75),      # 32 < N <= 256 router
    (600, 300, 128, 128, 1.0, 76),     # N > 256 router (logits in HBM)
    (4096, 64, 512, 1024, 1.0, 81),    # weight gradients on 256 x 256 tiles, operands K-outer
    (1500, 4, 128, 512, 1.0, 82),      # capacity 375: 256-row tiles from the tile list
])
def test_backward_shapes(B, T, N, d, F, c, seed):
    spec = S.Spec(f"bwd-{T}-{N}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, *_, f, g, G_bits = _run(B, spec)
    _check(spec, host, f, g, G_bits, 1.0, spec.name)


def test_backward_switch_base_shape(B):
    spec = S.CONFIGS[2]
    host, *_, f, g, G_bits = _run(B, spec, g_aux=3.0)
    _check(spec, host, f, g, G_bits, 3.0, "bwd-base")


def test_backward_one_expert_router_gets_nothing(B):
    """N = 1: the gate is 1 whatever the logits, so the router gradient is zero."""
    spec = S.Spec("bwd-n1", T=200, d=128, F=256, N=1, c=1.0, seed=77)
    host, *_, f, g, G_bits = _run(B, spec)
    assert np.all(g["grad_W_r"] == 0) and np.all(g["grad_b_r"] == 0)
    _check(spec, host, f, g, G_bits, 1.0, "bwd-n1")


def test_backward_capacity_zero_and_empty(B):
    """Every token dropped: expert gradients are zero, grad_x is G plus the
    router part of the loss; T = 0 writes zeros."""
    spec = S.Spec("bwd-c0", T=300, d=128, F=256, N=4, c=0.0, seed=78)
    host, *_, f, g, G_bits = _run(B, spec)
    assert np.all(g["grad_W_in"] == 0) and np.all(g["grad_W_out"] == 0)
    _check(spec, host, f, g, G_bits, 1.0, "bwd-c0")
    e = S.Spec("bwd-empty", T=0, d=128, F=128, N=4, c=1.0, seed=79)
    h0 = S.host_inputs(e.with_(T=1))
    layer = B.SwitchLayer.from_host(e, h0, t_max=8)
    fwd = layer.alloc(0)
    x = torch.empty((0, 128), dtype=torch.int16, device="cuda")
    layer.forward(x, 0, fwd)
    grads = layer.alloc_backward(0)
    for k in ("grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
        grads[k].fill_(7)
    layer.backward(x, 0, x, 1.0, fwd, grads)
    torch.cuda.synchronize()
    for k in ("grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
        assert int(grads[k].abs().sum().item()) == 0, k


def test_backward_deterministic(B):
    spec = S.Spec("bwd-det", T=1500, d=256, F=512, N=8, c=1.0, seed=80)
    host, layer, x, G, fwd, grads, f, g, _ = _run(B, spec)
    again = layer.alloc_backward(spec.T)
    layer.backward(x, spec.T, G, 1.0, fwd, again)
    torch.cuda.synchronize()
    for k in ("grad_x", "grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
        assert np.array_equal(B.from_device(again[k]), g[k]), k


@pytest.mark.parametrize("T,N,d,F,c,seed", [
    (1000, 8, 256, 512, 1.0, 91),      # several M tiles, drops of either choice
    (130, 16, 128, 256, 0.5, 92),      # heavy overflow: tokens with both choices dropped
    (700, 48, 128, 256, 1.0, 93),      # 32 < N <= 256 router
    (600, 300, 128, 128, 1.0, 94),     # N > 256 router (logits in HBM)
])
def test_backward_top2_shapes(B, T, N, d, F, c, seed):
    """Top-2 routing: two gated experts per token, loss term over k T assignments."""
    spec = S.Spec(f"bwd2-{T}-{N}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, *_, f, g, G_bits = _run(B, spec, g_aux=2.0, top_k=2)
    assert f["expert_idx"].shape == (T, 2)
    _check(spec, host, f, g, G_bits, 2.0, spec.name)


def test_backward_top2_switch_base_shape(B):
    spec = S.CONFIGS[2]
    host, *_, f, g, G_bits = _run(B, spec, top_k=2)
    _check(spec, host, f, g, G_bits, 1.0, "bwd2-base")


@pytest.mark.parametrize("top_k,T,N,d,F,c,seed", [
    (1, 1000, 8, 256, 512, 1.0, 95),
    (1, 4096, 64, 512, 1024, 1.0, 96),
    (2, 700, 48, 128, 256, 1.0, 97),
])
def test_backward_reads_forward_h(B, top_k, T, N, d, F, c, seed):
    """H taken from the forward call's workspace gives the gradients of the
    recomputation bit for bit; a forward workspace that is too small is refused."""
    spec = S.Spec(f"bwd-reuse-{top_k}-{T}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, layer, x, G, fwd, grads, f, g, G_bits = _run(B, spec, top_k=top_k)
    again = layer.alloc_backward(T)
    layer.backward(x, T, G, 1.0, fwd, again, reuse_forward=True)
    torch.cuda.synchronize()
    for k in ("grad_x", "grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
        assert np.array_equal(B.from_device(again[k]), g[k]), k
    a = again
    st = B.switch_backward(layer.handle, x, T, G, 1.0, fwd["logits"], fwd["expert_idx"],
                           fwd["gate"], fwd["position"], fwd["drop_mask"], fwd["load"],
                           a["grad_x"], a["grad_W_r"], a["grad_b_r"], a["grad_W_in"],
                           a["grad_W_out"], a["ws"], a["ws_bytes"], fwd["ws"],
                           fwd["ws_bytes"] - 1)
    assert st == B.SWITCH_E_INVALID


@pytest.mark.parametrize("T,N,d,F,c,seed", [
    (1000, 8, 256, 512, 1.0, 141),
    (2100, 16, 768, 512, 1.0, 142),
])
def test_backward_after_fused_forward(B, T, N, d, F, c, seed):
    """A forward on the fused FFN leaves no H in its workspace; a backward given that
    workspace recomputes H into it (its flag word says so) and gives the gradients of
    a backward without the workspace, bit for bit, then reads H from it the next time."""
    spec = S.Spec(f"bwd-fused-{T}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, layer, x, G, fwd, grads, f, g, G_bits = _run(B, spec)
    print(f"[case] backward after fused forward {spec.name}", flush=True)
    B.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_FUSED)
    fused = layer.alloc(T)
    layer.forward(x, T, fused)
    for k in ("expert_idx", "gate", "position", "drop_mask", "logits", "load"):
        assert np.array_equal(B.from_device(fused[k]), f[k]), k
    for rnd in range(2):
        again = layer.alloc_backward(T)
        layer.backward(x, T, G, 1.0, fused, again, reuse_forward=True)
        torch.cuda.synchronize()
        for k in ("grad_x", "grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
            assert np.array_equal(B.from_device(again[k]), g[k]), (rnd, k)


@pytest.mark.parametrize("top_k,T,N,d,F,c,seed", [
    (1, 4096, 8, 768, 3072, 1.25, 131),   # Switch-Base: split-K second matmul with the combine
    (1, 1000, 8, 256, 512, 1.0, 132),     # 128-row tiles
    (1, 4096, 64, 512, 1024, 1.0, 133),   # 64 experts
    (1, 9600, 32, 1024, 256, 1.0, 134),   # 256 x 256 second matmul with the combine
    (2, 700, 48, 128, 256, 1.0, 135),     # top-2: Y is always in the forward's buffer
])
def test_backward_reads_kept_y(B, top_k, T, N, d, F, c, seed):
    """A training forward (switch_set_keep_expert_out) gives the same outputs, and a
    backward given its workspace reads Y from it instead of recomputing it: the same
    gradients bit for bit.  A later forward that keeps nothing leaves the workspace
    marked so that the backward recomputes Y again."""
    spec = S.Spec(f"bwd-keep-y-{top_k}-{T}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, layer, x, G, fwd, grads, f, g, G_bits = _run(B, spec, top_k=top_k)
    print(f"[case] kept Y {spec.name}", flush=True)
    # the plain forward's outputs equal the training forward's bit for bit on the
    # two-launch FFN (a training forward always runs it)
    B.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_UNFUSED)
    layer.forward(x, T, fwd)
    keys = ("out", "expert_idx", "gate", "position", "drop_mask", "aux_loss", "logits", "load")
    plain = {k: B.from_device(fwd[k]) for k in keys}
    B.switch_set_keep_expert_out(layer.handle, True)
    kept = layer.alloc(T)
    layer.forward(x, T, kept)
    B.switch_set_keep_expert_out(layer.handle, False)
    torch.cuda.synchronize()
    for k in keys:
        assert np.array_equal(B.from_device(kept[k]), plain[k]), k
    again = layer.alloc_backward(T)
    B.switch_profile_enable(layer.handle, 1)
    layer.backward(x, T, G, 1.0, kept, again, reuse_forward=True)
    kept_stages = dict(B.switch_profile_read(layer.handle))
    B.switch_profile_enable(layer.handle, 0)
    torch.cuda.synchronize()
    for k in ("grad_x", "grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
        assert np.array_equal(B.from_device(again[k]), g[k]), k
    if top_k == 1 and T * d * F >= 4096 * 768 * 3072:
        # the gradients are the same either way, so tell a read of the kept Y from
        # a recomputation by time: the recomputation is a whole second matmul
        # (tens of microseconds here), while with Y kept its blocks exit at once
        layer.forward(x, T, fwd)   # keeps nothing: the shared workspace's flag is cleared
        B.switch_profile_enable(layer.handle, 1)
        layer.backward(x, T, G, 1.0, fwd, again, reuse_forward=True)
        fresh_stages = dict(B.switch_profile_read(layer.handle))
        B.switch_profile_enable(layer.handle, 0)
        assert kept_stages["recompute_y"] < 0.5 * fresh_stages["recompute_y"], \
            (kept_stages["recompute_y"], fresh_stages["recompute_y"])
    # the same workspace after a forward of another input that keeps nothing: its
    # buffer still holds the first input's Y, and the backward must recompute Y
    if top_k == 1:
        x2 = B.to_device(np.ascontiguousarray(host["x"][::-1]), layer.device)
        layer.forward(x2, T, kept)
        fresh = layer.alloc(T)
        layer.forward(x2, T, fresh)
        ref2 = layer.alloc_backward(T)
        layer.backward(x2, T, G, 1.0, fresh, ref2)
        third = layer.alloc_backward(T)
        layer.backward(x2, T, G, 1.0, kept, third, reuse_forward=True)
        torch.cuda.synchronize()
        for k in ("grad_x", "grad_W_r", "grad_b_r", "grad_W_in", "grad_W_out"):
            assert np.array_equal(B.from_device(third[k]), B.from_device(ref2[k])), k
    assert B.lib.switch_set_keep_expert_out(layer.handle, 2) == B.SWITCH_E_INVALID
    assert B.lib.switch_set_keep_expert_out(None, 1) == B.SWITCH_E_INVALID
