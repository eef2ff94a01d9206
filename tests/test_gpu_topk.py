"""GPU parity of the top-2 variant (classic MoE routing, the next row after the
Switch layer) against the CPU oracle's top-k routing and combine, through the C ABI.

Bars, as for top-1: routing stage (oracle top-k routing fed the GPU's fp32
logits) bit-exact for expert_idx, position, drop_mask and load, gate within
1e-6 relative, aux within 1e-5 relative; logits within the fp32 dot-product
bound; output within 1e-2 (1 + |ref|) of the oracle combine with the GPU's
routing; expert outputs (debug entry point) within 2^-6 (|E| + rms(E)).
"""
import numpy as np
import pytest

import oracle
import synthetic as S
import parity
from golden_util import keyed

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
K = 2


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from switch_transformer_top_amd import binding
    return binding


def _run(B, spec):
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, top_k=K)
    print(f"[case] top2 {spec.name} T={spec.T} d={spec.d} F={spec.F} N={spec.N} c={spec.c}",
          flush=True)
    res = layer.forward_host(host["x"], debug=True)
    plain = layer.forward_host(host["x"])
    for k in ("out", "expert_idx", "gate", "position", "drop_mask", "logits", "load"):
        assert np.array_equal(plain[k], res[k]), f"default path differs in {k}"
    return host, res


def _check_routing(res, spec, tag):
    ref = oracle.route_topk(res["logits"].astype(np.float64), K, spec.c, spec.capacity_override,
                            spec.alpha)
    assert res["expert_idx"].shape == (spec.T, K)
    for k, rk in (("expert_idx", "expert_idx"), ("position", "position"),
                  ("drop_mask", "drop"), ("load", "load")):
        assert np.array_equal(res[k], ref[rk]), f"{tag} {k}"
    rel = np.abs(res["gate"].astype(np.float64) - ref["gate"]) / ref["gate"]
    assert rel.max(initial=0) <= 1e-6, f"{tag} gate rel err {rel.max()}"
    arel = abs(res["aux_loss"] - ref["aux"]) / abs(ref["aux"])
    assert arel <= 1e-5, f"{tag} aux rel err {arel}"
    return ref


def _check_output(res, spec, host, tag):
    xf = S.to_f32(host["x"], spec.act)
    W_in = S.to_f32(host["W_in"], spec.expert)
    W_out = S.to_f32(host["W_out"], spec.expert)
    out_ref, E_ref = oracle.combine_topk(xf, res["expert_idx"], res["gate"].astype(np.float64),
                                         res["drop_mask"], W_in, W_out)
    out = S.to_f32(res["out"], spec.act).astype(np.float64)
    err = np.abs(out - out_ref)
    tol = 1e-2 * (1 + np.abs(out_ref))
    assert (err <= tol).all(), f"{tag} out err {(err - tol).max()}"
    # a token with both choices dropped leaves bit for bit
    gone = res["drop_mask"].all(axis=1)
    assert np.array_equal(res["out"][gone], host["x"][gone]), f"{tag} dropped rows changed"
    # expert outputs of the kept assignments, from the debug copy [N, Cb, d]
    kept = res["drop_mask"] == 0
    Cb = res["expert_out"].shape[1]
    e = res["expert_idx"][kept].astype(np.int64)
    p = res["position"][kept].astype(np.int64)
    got = S.to_f32(res["expert_out"].reshape(-1, spec.d)[e * Cb + p], spec.act).astype(np.float64)
    want = E_ref[kept]
    rms = np.sqrt(np.mean(want ** 2)) + 1e-30
    bad = np.abs(got - want) > 2.0 ** -6 * (np.abs(want) + rms)
    assert not bad.any(), f"{tag} expert output: {bad.sum()} elements off"


@pytest.mark.parametrize("T,N,d,F,c,seed,act", [
    (64, 4, 32, 64, 1.25, 51, "f32"),     # fp32 layer
    (1000, 8, 256, 512, 1.0, 52, "bf16"),  # several M tiles, drops
    (777, 5, 128, 384, 1.25, 53, "bf16"),  # odd expert count
    (130, 16, 128, 256, 0.5, 54, "bf16"),  # heavy overflow: both choices dropped for some tokens
    (9, 32, 128, 128, 2.0, 55, "bf16"),    # T < N
    (3000, 4, 128, 512, 1.0, 56, "bf16"),  # capacity >= 512: 256-row tiles
    (600, 300, 128, 128, 1.0, 57, "bf16"), # many experts: logits in HBM, statistics from them
    (700, 48, 128, 256, 1.0, 58, "bf16"),  # 32 < N <= 256: the token-split router
    (500, 1024, 128, 128, 2.0, 62, "bf16"),  # N = 1024: full 16-per-lane statistics rows
    (300, 1500, 128, 128, 2.0, 63, "bf16"),  # 1024 < N < 2048: 32 per lane, experts past N masked
    (400, 2048, 128, 128, 2.0, 65, "bf16"),  # N = 2048: full 32-per-lane rows with two choices
])
def test_top2_shapes(B, T, N, d, F, c, seed, act):
    spec = S.Spec(f"top2-{T}-{N}", T=T, d=d, F=F, N=N, c=c, seed=seed, act=act, expert=act)
    host, res = _run(B, spec)
    _check_routing(res, spec, spec.name)
    xf = S.to_f32(host["x"], spec.act)
    parity.check_logits(res["logits"], xf, host["W_r"], host["b_r"], tag=spec.name)
    _check_output(res, spec, host, spec.name)


def test_top2_switch_base_shape(B):
    """Switch-Base shapes (T = 4096, d = 768, F = 3072, 8 experts) routed top-2."""
    spec = S.CONFIGS[2]
    host, res = _run(B, spec)
    _check_routing(res, spec, "top2-base")
    _check_output(res, spec, host, "top2-base")


def test_top2_hospital_example_on_gpu(B):
    """llm-papers-study 3.1: softmax 0.6 / 0.3 / 0.1 -> experts 0 and 1, weights 0.6, 0.3."""
    g = keyed("lp_hospital_top2.txt")
    p = np.array(g["p"], dtype=np.float64)
    h = np.log(p)[None, :].astype(np.float32)
    spec = S.Spec("pin2", T=1, d=128, F=128, N=3, c=10.0, seed=59)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, top_k=K)
    bufs = layer.alloc(1)
    layer.route_from_logits(torch.from_numpy(h).cuda(), 1, bufs)
    torch.cuda.synchronize()
    assert B.from_device(bufs["expert_idx"]).tolist() == [[0, 1]]
    gates = B.from_device(bufs["gate"])[0]
    assert np.allclose(gates, g["top2_weights"], rtol=1e-6, atol=0)


def test_top2_ties_and_uniform_load_on_gpu(B):
    """Equal logits choose experts 0 and 1; a uniform assignment load gives aux = alpha."""
    spec = S.Spec("pin2b", T=40, d=128, F=128, N=4, c=1.0, seed=60)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host, top_k=K)
    bufs = layer.alloc(40)
    h = np.zeros((40, 4), np.float32)
    layer.route_from_logits(torch.from_numpy(h).cuda(), 40, bufs)
    torch.cuda.synchronize()
    assert np.all(B.from_device(bufs["expert_idx"]) == [0, 1])
    rng = np.random.default_rng(61)
    h = rng.uniform(-0.1, 0.1, size=(40, 4)).astype(np.float32)
    t = np.arange(40)
    h[t, t % 4] += 10.0
    h[t, (t + 1) % 4] += 5.0
    layer.route_from_logits(torch.from_numpy(h).cuda(), 40, bufs)
    torch.cuda.synchronize()
    assert np.all(B.from_device(bufs["load"]) == 20)
    assert float(bufs["aux_loss"].item()) == pytest.approx(spec.alpha, rel=1e-6)
