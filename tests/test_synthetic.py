"""The seeded input generator: determinism, slicing, distributions, bf16 rounding."""
import math

import numpy as np
import torch

import synthetic as S


def test_slices_regenerate_identically():
    full = S.fill(3, S.TENSOR_WIN, True, 0.02, 0, 5000, "bf16")
    part = S.fill(3, S.TENSOR_WIN, True, 0.02, 1234, 777, "bf16")
    assert np.array_equal(full[1234:1234 + 777], part)
    one = S.fill(3, S.TENSOR_WIN, True, 0.02, 4321, 1, "bf16", nthreads=1)
    assert one[0] == full[4321]


def test_streams_differ_by_seed_and_tensor():
    a = S.fill(1, 0, False, 1.0, 0, 1000, "f32")
    b = S.fill(2, 0, False, 1.0, 0, 1000, "f32")
    c = S.fill(1, 1, False, 1.0, 0, 1000, "f32")
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_normal_moments_and_truncation():
    z = S.fill(7, 0, False, 1.0, 0, 2_000_000, "f32").astype(np.float64)
    assert abs(z.mean()) < 3e-3 and abs(z.std() - 1) < 3e-3
    assert abs(np.mean(z ** 4) - 3.0) < 0.03                     # normal kurtosis
    tz = S.fill(7, 2, True, 1.0, 0, 2_000_000, "f32").astype(np.float64)
    assert tz.min() >= -2.0 and tz.max() <= 2.0
    # std of a standard normal truncated to [-2, 2]
    phi2 = math.exp(-2) / math.sqrt(2 * math.pi)
    mass = math.erf(2 / math.sqrt(2))
    assert abs(tz.std() - math.sqrt(1 - 4 * phi2 / mass)) < 3e-3


def test_bf16_is_round_to_nearest_even_of_the_float():
    f = S.fill(9, 3, True, 0.05, 0, 100_000, "f32")
    b = S.fill(9, 3, True, 0.05, 0, 100_000, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
    assert np.array_equal(S.bf16_to_f32(b), torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_log_helper_accuracy():
    lib = S._load_host()
    for s in np.geomspace(1e-30, 0.999999, 200):
        assert abs(lib.synth_ln_export(float(s)) - math.log(s)) <= 4e-16 * max(1.0, abs(math.log(s)))


def test_zipf_router_bias():
    spec = S.CONFIGS[3]
    b = S.router_bias(spec).astype(np.float64)
    s, beta = spec.zipf
    # b_i - b_j = beta * ln(p_i / p_j) = -beta * s * ln((i+1)/(j+1))
    assert abs((b[0] - b[9]) - beta * s * math.log(10)) < 1e-6
    assert np.all(np.diff(b) < 0)
    assert S.router_bias(S.CONFIGS[2]) is None


def test_config_shapes():
    assert [S.CONFIGS[i].T for i in range(1, 6)] == [64, 4096, 16384, 32768, 131072]
    assert S.CONFIGS[5].N * S.CONFIGS[5].F * S.CONFIGS[5].d * 2 * 2 == 103_079_215_104
