"""GPU parity of the HIP Switch layer against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synthetic as S
from golden_util import keyed, rows
import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from switch_transformer_top_amd import binding
    return binding


ROUTE_KEYS = ("expert_idx", "gate", "position", "drop_mask", "logits", "load")


def same_as_default_path(layer, x, res):
    """switch_forward (combine fused into the second matmul) must give the same
    bits as switch_forward_debug (expert output stored, separate combine pass)."""
    plain = layer.forward_host(x)
    for k in ("out",) + ROUTE_KEYS:
        assert np.array_equal(plain[k], res[k]), f"default path differs in {k}"
    assert plain["aux_loss"] == res["aux_loss"]


def _run(B, spec, host=None, debug=True):
    host = host or S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    # the debug entry point always runs the two-launch FFN; the bit-for-bit
    # comparison with the default path holds on that path
    B.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_UNFUSED)
    print(f"[case] {spec.name} T={spec.T} d={spec.d} F={spec.F} N={spec.N} c={spec.c}", flush=True)
    res = layer.forward_host(host["x"], debug=debug)
    if debug:
        same_as_default_path(layer, host["x"], res)
    return host, layer, res


def _full_check(spec, host, res, tag):
    parity.check_routing_stage(res, spec, tag)
    xf = S.to_f32(host["x"], spec.act)
    h_ref = parity.check_logits(res["logits"], xf, host["W_r"], host["b_r"], tag=tag)
    parity.check_end_to_end(res, h_ref, spec, tag=tag)
    parity.check_output_full(res, spec, host, tag)


# ---------------------------------------------------------------- workloads

def test_tiny_fp32_config(B):
    spec = S.CONFIGS[1]
    host, _, res = _run(B, spec)
    assert int(res["drop_mask"].sum()) >= 0
    _full_check(spec, host, res, "tiny-fp32")


@pytest.mark.parametrize("T,N,d,F,c,seed", [
    (1000, 8, 256, 512, 1.0, 21),      # ragged T, several M tiles, drops
    (777, 5, 128, 384, 1.25, 22),      # odd expert count
    (130, 16, 128, 256, 0.5, 23),      # heavy overflow
    (64, 1, 128, 128, 1.0, 24),        # one expert: gate 1, aux alpha
    (9, 32, 128, 128, 2.0, 25),        # T < N
    (3000, 4, 128, 512, 1.0, 26),      # capacity >= 512: 256-row tiles, three M tiles
    (2100, 4, 256, 768, 1.0, 27),      # 256-row tiles with a ragged last tile and drops
    (1500, 4, 128, 512, 1.0, 28),      # capacity 375: one full 256-row tile and a ragged one
    (9600, 32, 1024, 256, 1.0, 29),    # capacity 300: second matmul on 256-row tiles, combine fused
    (8192, 256, 256, 256, 1.0, 30),    # capacity 32 with more tiles than CUs: 64-row tiles
    (1000, 520, 128, 256, 1.0, 31),    # logits router: three expert tiles (the last of 8), a
                                       # 256-token block whose second 128-token group is partial
    (1300, 1500, 128, 128, 2.0, 35),   # 1024 < N < 2048: the 32-per-lane statistics with the
                                       # experts past N masked, a ragged last expert tile
    (1000, 600, 1024, 256, 1.0, 36),   # logits router over 32 K steps: the x ring refilled
                                       # three steps ahead, a ragged last expert tile
    (300, 300, 2048, 128, 1.0, 37),    # the 2048-wide rows of the 2048-expert share (64 K
                                       # steps), one partial token tile
    (700, 2048, 128, 128, 1.0, 38),    # N = 2048: full 32-per-lane statistics rows, a ragged
                                       # last chunk of 60 tokens
    (640, 512, 128, 128, 1.0, 39),     # N = 512: full 8-per-lane rows, whole chunks only
    (600, 1024, 128, 256, 1.0, 41),    # N = 1024: full 16-per-lane rows
])
def test_bf16_ragged_shapes(B, T, N, d, F, c, seed):
    spec = S.Spec(f"bf16-{T}-{N}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, _, res = _run(B, spec)
    _full_check(spec, host, res, spec.name)
    if N == 1:
        assert np.all(res["gate"] == 1.0)
        assert res["aux_loss"] == pytest.approx(spec.alpha, rel=1e-6)


def test_more_than_2048_experts(B):
    """N = 3000 (create accepts up to 8192) takes the statistics kernel that walks each
    logit row in pieces (more than 32 logits per lane): the layer end to end against
    the oracle, then the routing stage alone from the same logits through
    switch_route_from_logits, which must give the same bits."""
    spec = S.Spec("bf16-2000-3000", T=2000, d=128, F=128, N=3000, c=1.0, seed=34)
    host, layer, res = _run(B, spec)
    _full_check(spec, host, res, spec.name)
    bufs = layer.alloc(spec.T)
    hl = torch.from_numpy(np.ascontiguousarray(res["logits"])).cuda()
    print(f"[case] route_from_logits N={spec.N}", flush=True)
    layer.route_from_logits(hl, spec.T, bufs)
    torch.cuda.synchronize()
    for k in ("expert_idx", "gate", "position", "drop_mask", "load"):
        assert np.array_equal(B.from_device(bufs[k]), res[k]), k
    assert float(bufs["aux_loss"].item()) == res["aux_loss"]


def test_logits_router_bias_odd_width(B):
    """N = 777 with a router bias: the many-expert logits router stores rows whose width is
    not a multiple of 4 (element stores past each 4-wide piece's end are left out), adds the
    bias in its staged epilogue, and ends in a partial expert tile (9 experts) and a
    partial token tile (132 tokens); the statistics kernel masks the experts past N."""
    spec = S.Spec("bf16-900-777-bias", T=900, d=128, F=128, N=777, c=1.25, seed=64,
                  zipf=(1.1, 0.12))
    host, _, res = _run(B, spec)
    assert host["b_r"] is not None
    _full_check(spec, host, res, spec.name)


# ---------------------------------------------------------------- fused expert FFN

def _run_fused(B, spec, host=None):
    """Forward with the fused expert FFN (H on chip); the profiler's stage names
    show that it ran."""
    host = host or S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    B.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_FUSED)
    print(f"[case] fused {spec.name} T={spec.T} d={spec.d} F={spec.F} N={spec.N} c={spec.c}",
          flush=True)
    B.switch_profile_enable(layer.handle, 1)
    res = layer.forward_host(host["x"])
    stages = [n for n, _ in B.switch_profile_read(layer.handle)]
    B.switch_profile_enable(layer.handle, 0)
    if spec.T > 0 and res["drop_mask"].min() == 0:   # some token reaches an expert
        assert "ffn_fused" in stages and "gemm1_relu" not in stages, stages
    return host, layer, res


@pytest.mark.parametrize("T,N,d,F,c,seed", [
    (1000, 8, 256, 512, 1.0, 41),      # one output tile per wave, two hidden chunks, ragged rows
    (777, 5, 512, 768, 1.25, 42),      # two output tiles per wave, three chunks, odd expert count
    (2100, 16, 768, 256, 1.0, 43),     # three output tiles per wave (Switch-Base width), one chunk
    (1500, 12, 1024, 512, 1.0, 44),    # four output tiles per wave (Switch-Large width)
    (130, 16, 256, 256, 0.5, 45),      # heavy overflow: dropped rows copied by the slot kernel
    (64, 1, 256, 256, 1.0, 46),        # one expert
    (9, 32, 256, 256, 2.0, 47),        # T < N: most experts empty
    (3000, 300, 256, 512, 1.0, 48),    # logits router: scan and slot kernels build the tile list
])
def test_fused_ffn_shapes(B, T, N, d, F, c, seed):
    spec = S.Spec(f"fused-{T}-{N}-{d}", T=T, d=d, F=F, N=N, c=c, seed=seed)
    host, _, res = _run_fused(B, spec)
    _full_check(spec, host, res, spec.name)
    if N == 1:
        assert np.all(res["gate"] == 1.0)


def test_fused_ffn_capacity_zero(B):
    spec = S.Spec("fused-c0", T=300, d=256, F=256, N=4, c=0.0, seed=49)
    host, _, res = _run_fused(B, spec)
    assert np.all(res["drop_mask"] == 1)
    assert np.array_equal(res["out"], host["x"])


def test_fused_ffn_switch_base_and_zipf(B):
    for cfg in (2, 3):
        spec = S.CONFIGS[cfg]
        host, layer, res = _run_fused(B, spec)
        _full_check(spec, host, res, f"fused-{spec.name}")
        # routing does not depend on the FFN variant
        B.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_UNFUSED)
        two = layer.forward_host(host["x"])
        for k in ROUTE_KEYS:
            assert np.array_equal(two[k], res[k]), k
        assert np.array_equal(two["out"][res["drop_mask"] == 1], res["out"][res["drop_mask"] == 1])


def test_ffn_mode_arguments(B):
    spec = S.Spec("mode", T=64, d=128, F=256, N=4, c=1.0, seed=50)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    assert B.lib.switch_set_ffn_mode(layer.handle, 3) == B.SWITCH_E_INVALID
    assert B.lib.switch_set_ffn_mode(None, 0) == B.SWITCH_E_INVALID
    # d = 128 is not a multiple of 256: the fused kernel does not take it
    assert B.lib.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_FUSED) == B.SWITCH_E_UNSUPPORTED
    assert B.lib.switch_set_ffn_mode(layer.handle, B.SWITCH_FFN_UNFUSED) == B.SWITCH_OK


def test_switch_base_config_full(B):
    spec = S.CONFIGS[2]
    host, _, res = _run(B, spec)
    _full_check(spec, host, res, "switch-base")


def test_zipf_overflow_config_full(B):
    spec = S.CONFIGS[3]
    host, _, res = _run(B, spec)
    _full_check(spec, host, res, "zipf")
    assert res["drop_mask"].mean() > 0.3        # the Zipf bias overflows popular experts
    assert (res["load"] < 0.25 * 128).sum() > 20  # and leaves many experts nearly empty


# ---------------------------------------------------------------- edge cases

def test_zero_tokens(B):
    spec = S.Spec("empty", T=0, d=128, F=128, N=4, c=1.0, seed=30)
    host = S.host_inputs(spec.with_(T=1))
    layer = B.SwitchLayer.from_host(spec, host, t_max=8)
    bufs = layer.alloc(0)
    bufs["aux_loss"].fill_(123.0)
    bufs["load"].fill_(-5)
    x = torch.empty((0, 128), dtype=torch.int16, device="cuda")
    layer.forward(x, 0, bufs)
    torch.cuda.synchronize()
    assert float(bufs["aux_loss"].item()) == 0.0
    assert int(bufs["load"].abs().sum().item()) == 0


def test_capacity_zero_passes_everything_through(B):
    spec = S.Spec("c0", T=300, d=128, F=256, N=4, c=0.0, seed=31)
    host, _, res = _run(B, spec)
    assert np.all(res["drop_mask"] == 1)
    assert np.array_equal(res["out"], host["x"])
    parity.check_routing_stage(res, spec, "c0")


def test_large_capacity_drops_nothing(B):
    spec = S.Spec("cN", T=500, d=128, F=256, N=4, c=4.0, seed=32)
    host, _, res = _run(B, spec)
    assert not res["drop_mask"].any()
    _full_check(spec, host, res, "cN")


def test_deterministic_bitwise(B):
    spec = S.Spec("det", T=2000, d=256, F=512, N=16, c=1.0, seed=33)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    a = layer.forward_host(host["x"])
    b = layer.forward_host(host["x"])
    for k in ("out",) + ROUTE_KEYS:
        assert np.array_equal(a[k], b[k]), k
    assert a["aux_loss"] == b["aux_loss"]


# ---------------------------------------------------------------- pinned examples through the GPU

def _route_logits(B, h: np.ndarray, c: float, capacity_override: int = 0):
    """GPU routing stage (switch_route_from_logits) on given fp32 logits."""
    T, N = h.shape
    spec = S.Spec("pin", T=T, d=128, F=128, N=N, c=c, seed=40, capacity_override=capacity_override)
    host = S.host_inputs(spec)
    layer = B.SwitchLayer.from_host(spec, host)
    bufs = layer.alloc(T)
    hl = torch.from_numpy(np.ascontiguousarray(h, dtype=np.float32)).cuda()
    layer.route_from_logits(hl, T, bufs)
    torch.cuda.synchronize()
    r = {k: B.from_device(bufs[k]) for k in ("expert_idx", "gate", "position", "drop_mask", "load")}
    r["aux_loss"] = float(bufs["aux_loss"].item())
    r["logits"] = h.astype(np.float32)
    return r, spec


def test_pin_softmax_table_on_gpu(B):
    tab = np.array([[float(v) for v in r] for r in rows("ms_softmax_table.txt")])
    p, sel = tab[:, :4], tab[:, 4].astype(np.int32)
    h = np.log(np.where(p > 0, p, 1e-12)).astype(np.float32)
    r, spec = _route_logits(B, h, c=1.0)
    assert np.array_equal(r["expert_idx"], sel)
    assert list(r["drop_mask"]) == [0, 0, 1, 1, 0]
    assert r["aux_loss"] == pytest.approx(0.01 * 4 * 0.472, rel=1e-5)
    parity.check_routing_stage(r, spec, "softmax-table")


def test_pin_sixteen_tokens_on_gpu(B):
    g = keyed("kb_capacity_16_4.txt")
    rng = np.random.default_rng(5)
    perm = rng.permutation(np.repeat(np.arange(4), g["loads"]))
    h = rng.uniform(-0.1, 0.1, size=(16, 4))
    h[np.arange(16), perm] += 10.0
    r, spec = _route_logits(B, h.astype(np.float32), c=g["c"])
    assert list(r["load"]) == g["loads"]
    assert int(r["drop_mask"].sum()) == g["overflow_count"]
    assert set(perm[r["drop_mask"].astype(bool)]) == {g["overflow_expert"]}
    parity.check_routing_stage(r, spec, "sixteen")


def test_pin_ties_and_uniform_aux_on_gpu(B):
    r, spec = _route_logits(B, np.zeros((50, 8), np.float32), c=1.0)
    assert np.all(r["expert_idx"] == 0)
    assert np.allclose(r["gate"], 1 / 8, rtol=1e-7)
    assert r["aux_loss"] == pytest.approx(0.01, rel=1e-6)
    h = np.full((3, 6), -1.0, np.float32)
    h[:, 2] = h[:, 4] = 2.0
    r, _ = _route_logits(B, h, c=1.0)
    assert np.all(r["expert_idx"] == 2)


def test_pin_hand_example_on_gpu(B):
    """The overflowing token passes through unchanged (byhand.ai steps 7 and 13).
    fp32 layer, d padded with zero features to the library's multiple of 8."""
    g = keyed("bh_hand_example.txt")
    d = F = 8
    W_r = np.zeros((3, d), np.float32)
    W_r[:, :3] = [[0, 0, 2], [0, 1, 0], g["switch_row_C"]]
    x = np.zeros((5, d), np.float32)
    x[:, :3] = [[0, 0, 3], [0, 2, 1], [0, 3, -1], [0, 3, 1], g["Z5"]]
    rng = np.random.default_rng(0)
    W_in = rng.normal(0, 0.5, size=(3, F, d)).astype(np.float32)
    W_out = rng.normal(0, 0.5, size=(3, d, F)).astype(np.float32)
    spec = S.Spec("hand", T=5, d=d, F=F, N=3, c=1.0, act="f32", expert="f32")
    host = dict(x=x, W_r=W_r, b_r=None, W_in=W_in, W_out=W_out)
    _, _, res = _run(B, spec, host)
    assert list(res["expert_idx"]) == [0, 2, 1, 2, 2]
    assert res["drop_mask"][4] == 1 and res["position"][4] == g["capacity"]
    assert np.array_equal(res["out"][4], x[4])
    _full_check(spec, host, res, "hand")
