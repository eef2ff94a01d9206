"""Pins of the oracle's backward pass (no GPU).

The backward is the chain rule on the forward's definition, with the expert
choice and the capacity cut held fixed (the kasblo explainer, section
"argmaxは離散なのに、Routerはなぜ学習できるのか": the discrete choice gives no
gradient, the continuous gate p_{i*}(x) carries it to the softmax and W_r;
llm-papers-study section 3.3: f_i is discrete, P_i continuous).  It is pinned
to things other than itself:
  - central finite differences of the oracle's forward (a different code path)
    for every input, at a routing the perturbation cannot change;
  - torch's CPU autograd (float64) for the one-expert layer, a dense MLP;
  - the closed form of the softmax Jacobian on one token.
"""
import numpy as np
import pytest

import oracle

ALPHA = 0.01
EPS = 2.0 ** -12      # exact in float32 for inputs on a 2^-8 grid


def _grid(rng, shape, scale=1.0):
    """Values on a 2^-8 grid, so value +- EPS stays exact in float32."""
    return (np.round(rng.standard_normal(shape) * scale * 256) / 256).astype(np.float32)


def _problem(seed, T=7, d=4, F=5, N=3, c=0.8):
    rng = np.random.default_rng(seed)
    x = _grid(rng, (T, d))
    W_r = _grid(rng, (N, d), 1.5)
    b_r = _grid(rng, (N,), 0.5)
    W_in = _grid(rng, (N, F, d))
    W_out = _grid(rng, (N, d, F))
    G = rng.standard_normal((T, d))
    return x, W_r, b_r, W_in, W_out, G, c


def _loss(x, W_r, b_r, W_in, W_out, G, c, g_aux):
    r = oracle.forward(x, W_r, b_r, W_in, W_out, c, alpha=ALPHA)
    return float((G * r["out"]).sum() + g_aux * r["aux"]), r


def _stable(x, W_r, b_r, W_in, W_out, c):
    """True when no logit margin or ReLU input is within reach of the perturbation."""
    r = oracle.forward(x, W_r, b_r, W_in, W_out, c, alpha=ALPHA)
    h = r["h"]
    part = np.sort(h, axis=1)
    if (part[:, -1] - part[:, -2]).min() < 0.05:
        return False
    for t in range(x.shape[0]):
        u = W_in[r["expert_idx"][t]].astype(np.float64) @ x[t].astype(np.float64)
        if np.abs(u).min() < 0.05:
            return False
    return True


def _backward(x, W_r, b_r, W_in, W_out, G, c, g_aux):
    r = oracle.forward(x, W_r, b_r, W_in, W_out, c, alpha=ALPHA)
    return oracle.backward(x, W_r, W_in, W_out, r["h"], r["expert_idx"], r["gate"], r["drop"],
                           r["load"], G, g_aux, ALPHA), r


@pytest.mark.parametrize("seed,g_aux", [(1, 0.0), (2, 1.0), (3, 7.5), (4, 1.0)])
def test_backward_matches_finite_differences(seed, g_aux):
    for s in range(seed, seed + 200, 4):       # the first seed whose routing is stable
        prob = _problem(s)
        if _stable(*prob[:5], prob[6]):
            break
    else:
        pytest.skip("no stable problem found")
    x, W_r, b_r, W_in, W_out, G, c = prob
    grads, r = _backward(x, W_r, b_r, W_in, W_out, G, c, g_aux)
    assert r["drop"].any() and not r["drop"].all()     # both branches are exercised

    def fd(arr, name):
        out = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + EPS
            lp, rp = _loss(x, W_r, b_r, W_in, W_out, G, c, g_aux)
            arr[idx] = keep - EPS
            lm, rm = _loss(x, W_r, b_r, W_in, W_out, G, c, g_aux)
            arr[idx] = keep
            assert np.array_equal(rp["expert_idx"], r["expert_idx"]), name
            assert np.array_equal(rm["drop"], r["drop"]), name
            out[idx] = (lp - lm) / (2 * EPS)
        return out

    for name, arr, got in (("x", x, grads["dx"]), ("W_r", W_r, grads["dW_r"]),
                           ("b_r", b_r, grads["db"]), ("W_in", W_in, grads["dW_in"]),
                           ("W_out", W_out, grads["dW_out"])):
        want = fd(arr, name)
        assert np.allclose(got, want, rtol=1e-6, atol=1e-7), \
            f"{name}: max err {np.abs(got - want).max()}"


def test_one_expert_layer_matches_torch_autograd():
    """N = 1: gate = 1 and the router gets no gradient; the layer is
    x + W_out relu(W_in x), whose gradients torch's autograd gives."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    T, d, F = 12, 6, 10
    x = rng.standard_normal((T, d)).astype(np.float32)
    W_in = rng.standard_normal((1, F, d)).astype(np.float32)
    W_out = rng.standard_normal((1, d, F)).astype(np.float32)
    W_r = rng.standard_normal((1, d)).astype(np.float32)
    G = rng.standard_normal((T, d))
    grads, r = _backward(x, W_r, None, W_in, W_out, G, 2.0, 1.0)
    assert not r["drop"].any()
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wi = torch.tensor(W_in[0], dtype=torch.float64, requires_grad=True)
    wo = torch.tensor(W_out[0], dtype=torch.float64, requires_grad=True)
    out = xt + torch.relu(xt @ wi.T) @ wo.T
    (out * torch.tensor(G)).sum().backward()
    assert np.allclose(grads["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(grads["dW_in"][0], wi.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(grads["dW_out"][0], wo.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(grads["dW_r"] == 0) and np.all(grads["db"] == 0)


def test_router_gradient_is_the_softmax_jacobian():
    """One kept token, no loss term: dh_i = p_e s (delta_ie - p_i) with s = G . E
    (the derivative of the gate p_e with respect to the logits, times G . E)."""
    rng = np.random.default_rng(31)
    d, F, N = 5, 7, 4
    x = rng.standard_normal((1, d)).astype(np.float32)
    W_r = rng.standard_normal((N, d)).astype(np.float32)
    W_in = rng.standard_normal((N, F, d)).astype(np.float32)
    W_out = rng.standard_normal((N, d, F)).astype(np.float32)
    G = rng.standard_normal((1, d))
    grads, r = _backward(x, W_r, None, W_in, W_out, G, 4.0, 0.0)
    e = int(r["expert_idx"][0])
    h = r["h"][0]
    p = np.exp(h - h.max()) / np.exp(h - h.max()).sum()
    s = float(G[0] @ r["E"][0])
    dh = p[e] * s * ((np.arange(N) == e) - p)
    assert np.allclose(grads["db"], dh, rtol=1e-12, atol=1e-14)
    assert np.allclose(grads["dW_r"], np.outer(dh, x[0].astype(np.float64)), rtol=1e-12,
                       atol=1e-14)


def test_loss_gradient_flows_through_p_only():
    """G = 0: only the loss moves the router, through P (f is a count); for token
    t, dh = (alpha N / T) p * (f - p . f)."""
    x, W_r, b_r, W_in, W_out, _, c = _problem(41, T=9, N=4)
    G = np.zeros((9, 4))
    grads, r = _backward(x, W_r, b_r, W_in, W_out, G, c, 1.0)
    T, N = 9, 4
    f = r["load"] / T
    h = r["h"]
    p = np.exp(h - h.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dh = (ALPHA * N / T) * p * (f[None, :] - (p * f[None, :]).sum(axis=1, keepdims=True))
    assert np.allclose(grads["db"], dh.sum(axis=0), rtol=1e-12, atol=1e-15)
    assert np.all(grads["dW_in"] == 0) and np.all(grads["dW_out"] == 0)


# ---------------------------------------------------------------------------
# top-k (k = 2): the same chain rule with two gated experts per token


def _loss_topk(x, W_r, b_r, W_in, W_out, G, c, g_aux, k):
    h = oracle.logits(x, W_r, b_r)
    r = oracle.route_topk(h, k, c, alpha=ALPHA)
    out, _ = oracle.combine_topk(x, r["expert_idx"], r["gate"], r["drop"], W_in, W_out)
    return float((G * out).sum() + g_aux * r["aux"]), r, h


def _stable_topk(x, W_r, b_r, W_in, W_out, c, k):
    """Margins between the k + 1 largest logits and the chosen experts' ReLU
    inputs all clear of the perturbation."""
    _, r, h = _loss_topk(x, W_r, b_r, W_in, W_out, np.zeros_like(x, dtype=np.float64), c, 0.0,
                         k)
    part = np.sort(h, axis=1)[:, ::-1]
    if (part[:, :k] - part[:, 1:k + 1]).min() < 0.05:
        return False
    for t in range(x.shape[0]):
        for j in range(k):
            u = W_in[r["expert_idx"][t, j]].astype(np.float64) @ x[t].astype(np.float64)
            if np.abs(u).min() < 0.05:
                return False
    return True


@pytest.mark.parametrize("seed,g_aux", [(5, 0.0), (6, 1.0), (7, 3.0)])
def test_topk_backward_matches_finite_differences(seed, g_aux):
    k = 2
    for s in range(seed, seed + 400, 4):
        prob = _problem(s, T=7, d=4, F=5, N=4, c=0.7)
        if _stable_topk(*prob[:5], prob[6], k):
            break
    else:
        pytest.skip("no stable problem found")
    x, W_r, b_r, W_in, W_out, G, c = prob
    _, r, h = _loss_topk(x, W_r, b_r, W_in, W_out, G, c, g_aux, k)
    assert r["drop"].any() and not r["drop"].all()     # both branches are exercised
    grads = oracle.backward_topk(x, W_r, W_in, W_out, h, r["expert_idx"], r["gate"], r["drop"],
                                 r["load"], G, g_aux, ALPHA)

    def fd(arr, name):
        out = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + EPS
            lp, rp, _ = _loss_topk(x, W_r, b_r, W_in, W_out, G, c, g_aux, k)
            arr[idx] = keep - EPS
            lm, rm, _ = _loss_topk(x, W_r, b_r, W_in, W_out, G, c, g_aux, k)
            arr[idx] = keep
            assert np.array_equal(rp["expert_idx"], r["expert_idx"]), name
            assert np.array_equal(rm["drop"], r["drop"]), name
            out[idx] = (lp - lm) / (2 * EPS)
        return out

    for name, arr, got in (("x", x, grads["dx"]), ("W_r", W_r, grads["dW_r"]),
                           ("b_r", b_r, grads["db"]), ("W_in", W_in, grads["dW_in"]),
                           ("W_out", W_out, grads["dW_out"])):
        want = fd(arr, name)
        assert np.allclose(got, want, rtol=1e-6, atol=1e-7), \
            f"{name}: max err {np.abs(got - want).max()}"


def test_topk_backward_at_one_choice_is_the_top1_backward():
    """k = 1: the same gradients as the top-1 backward."""
    x, W_r, b_r, W_in, W_out, G, c = _problem(51, T=9, N=3)
    grads1, r = _backward(x, W_r, b_r, W_in, W_out, G, c, 2.0)
    gk = oracle.backward_topk(x, W_r, W_in, W_out, r["h"], r["expert_idx"][:, None],
                              r["gate"][:, None], r["drop"][:, None], r["load"], G, 2.0, ALPHA)
    for key in ("dx", "dW_r", "db", "dW_in", "dW_out"):
        assert np.allclose(gk[key], grads1[key], rtol=1e-13, atol=1e-15), key
