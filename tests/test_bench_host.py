"""Host logic of the measurement (bench.py), no GPU: the per-stage work model
against the formulas of the measurement plan, the roofline bound choice, the
traffic lookup in the committed counter profiles and its source check, the load
summary, and the one-GPU guard."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synthetic as S


def test_gemm_work_matches_the_plan():
    # expert FLOPs count kept rows only: 4 kept d F over the two matmuls
    spec = S.CONFIGS[2]
    kept, active = 4000, 8
    w1 = bench.stage_work("gemm1_relu", spec, kept, active)
    w2 = bench.stage_work("gemm2_combine", spec, kept, active)
    assert w1["flops"] + w2["flops"] == 4.0 * kept * spec.d * spec.F
    # weights of the experts in use plus the kept rows' activations (bf16)
    assert w1["bytes"] == active * spec.d * spec.F * 2 + kept * (spec.d + spec.F) * 2
    # the fused combine adds the residual rows, the output rows and gate + slot
    assert w2["bytes"] == active * spec.d * spec.F * 2 + kept * (spec.F + 2 * spec.d) * 2 + 8 * kept


def test_mover_and_router_work_match_the_plan():
    spec = S.CONFIGS[5]
    T, d, N = spec.T, spec.d, spec.N
    kept = T - 9804
    # combine: (kept + 2T) d 2 + 13 T
    assert bench.stage_work("combine", spec, kept, N)["bytes"] == (kept + 2 * T) * d * 2 + 13 * T
    # the slot kernel of the bf16 top-1 path: dropped rows copied, 21 bytes per token
    assert bench.stage_work("dispatch", spec, kept, N)["bytes"] == 2 * (T - kept) * d * 2 + 21 * T
    # logits router: x, W_r, 8 bytes per token and the logits; three bf16 passes
    w = bench.stage_work("router_logits", spec, kept, N)
    assert w["bytes"] == T * d * 2 + N * d * 4 + 8 * T + T * N * 4
    assert w["flops"] == 3 * 2.0 * T * d * N
    assert bench.stage_work("route_rows", spec, kept, N)["bytes"] == T * N * 4 + 8 * T


def test_roofline_bound_and_fraction():
    # a contraction whose MFMA time exceeds its HBM time is MFMA-bound
    e = bench.roofline_entry("x", dict(flops=2.5e12, bytes=1e9, peak_tflops=2500.0), 2.0)
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s"
    assert e["achieved"] == pytest.approx(1250.0) and e["frac"] == pytest.approx(0.5)
    # and a stream with few flops per byte is HBM-bound
    e = bench.roofline_entry("y", dict(flops=1e9, bytes=8e9, peak_tflops=2500.0), 2.0)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s"
    assert e["achieved"] == pytest.approx(4000.0) and e["frac"] == pytest.approx(0.5)
    # movers have no flops
    e = bench.roofline_entry("z", dict(flops=0.0, bytes=4e9, peak_tflops=None), 1.0)
    assert e["bound"] == "hbm" and e["mfma_frac"] is None


def _fake_tree(tmp_path, text):
    csrc = tmp_path / "switch_transformer_top_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f, body in (("gemm.hip", text), ("common.hpp", "c"), ("epilogue.hpp", "e")):
        (csrc / f).write_text(body)
    (tmp_path / "profiles").mkdir()
    h = hashlib.sha256()
    for body in (text, "c", "e"):
        h.update(body.encode())
    return h.hexdigest()


def test_traffic_lookup_needs_matching_source(tmp_path, monkeypatch):
    digest = _fake_tree(tmp_path, "kernel v1")
    line = ("traffic: workload=wl kernel=gemm_bf16_kernel<64, 128, true, 1> "
            f"bytes_per_launch=123456 source=gemm.hip source_sha256={digest}\n")
    (tmp_path / "profiles" / "x_hbm_bytes.md").write_text("# t\n\n" + line)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gemm1_relu", "wl") == 123456.0
    assert bench.measured_traffic("gemm1_relu", "other") is None      # other workload
    assert bench.measured_traffic("gemm2_combine", "wl") is None      # other kernel
    # the kernel source changed since the counters were taken: no figure
    (tmp_path / "switch_transformer_top_amd" / "csrc" / "gemm.hip").write_text("kernel v2")
    assert bench.measured_traffic("gemm1_relu", "wl") is None


def test_committed_traffic_lines_parse():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    n = 0
    for f in os.listdir(os.path.join(root, "profiles")):
        if f.endswith("_hbm_bytes.md"):
            for line in open(os.path.join(root, "profiles", f), encoding="utf-8"):
                if line.startswith("traffic:"):
                    m = bench._TRAFFIC_LINE.match(line)
                    assert m, line
                    assert int(m["bytes_per_launch"]) > 0
                    n += 1
    assert n > 0


def test_load_summary():
    load = np.array([0, 3, 7, 7, 100, 2], dtype=np.int32)
    s = bench.load_summary(load, 5)
    assert s["min"] == 0 and s["max"] == 100
    assert s["empty_experts"] == 1 and s["over_capacity"] == 3
    assert s["top8"][:3] == [100, 7, 7]


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
