"""Benchmark of the Switch FFN layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

One step = one switch_forward call over the whole workload (router, softmax and
top-1, capacity assignment, load-balancing loss, dispatch, both expert matmuls,
combine) on seeded synthetic inputs already resident in HBM.  The default
workload is the Switch-Base-shaped layer: T=4096 tokens, d_model=768,
d_ff=3072, 8 experts, capacity factor 1.25.

Prints one JSON line: routed tokens/s over K timed steps; the roofline of the
dominant kernel (algorithmic work per launch / its mean duration from HIP
events the library records on its own stream over a second pass of K steps);
and the CPU oracle's throughput on the host cores.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as S  # noqa: E402

METRIC = "Switch-FFN fwd routed tokens/s (bf16); % MFMA peak & dispatch % HBM BW"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# workloads whose weight banks are written into HBM by the device generator
DEVICE_WEIGHTS = {4, 5}


def stage_work(stage: str, spec, kept: int, active_experts: int, k: int = 1) -> dict:
    """Algorithmic FLOPs and HBM bytes one launch of a stage must do (kept counts
    assignments: tokens at top-1, token-expert pairs at top-2)."""
    T, d, F, N = spec.T, spec.d, spec.F, spec.N
    es = 2 if spec.act == "bf16" else 4
    if stage in ("router", "router_logits"):
        # fp32 logits of bf16 tokens run as three exact bf16 MFMA passes (one per
        # piece of the split fp32 weight); fp32 tokens run on the fp32 FMA units.
        # The router reads x and W_r and writes the per-token routing results.
        nbytes = T * d * es + N * d * 4 + 8 * T + (T * N * 4 if stage == "router_logits" else 0)
        if spec.act == "bf16":
            return dict(flops=3 * 2.0 * T * d * N, bytes=nbytes, peak_tflops=PEAK_BF16_TFLOPS)
        return dict(flops=2.0 * T * d * N, bytes=nbytes, peak_tflops=PEAK_FP32_TFLOPS)
    peak = PEAK_BF16_TFLOPS if spec.expert == "bf16" else PEAK_FP32_TFLOPS
    if stage in ("gemm1_relu", "gemm2"):
        # weights of the experts in use, the kept rows in and the outputs out
        return dict(flops=2.0 * kept * d * F,
                    bytes=active_experts * d * F * es + kept * (d + F) * es, peak_tflops=peak)
    if stage == "gemm2_combine":
        # as gemm2, plus the residual rows read and the layer output written in
        # place of the expert output (gate and slot table: 8 bytes per row)
        return dict(flops=2.0 * kept * d * F,
                    bytes=active_experts * d * F * es + kept * (F + 2 * d) * es + 8 * kept,
                    peak_tflops=peak)
    if stage in ("dispatch", "assign"):
        # assign: the one-launch form (chunk scan and loss included; their
        # per-chunk counts are a few bytes per token and are left out)
        if spec.act == "bf16":
            # slot table only (the rows stay in place); at top-1 dropped rows copied to out
            rows = 2 * (T - kept) * d * es if k == 1 else 0
            return dict(flops=0.0, bytes=rows + (13 * k + 8) * T, peak_tflops=None)
        return dict(flops=0.0, bytes=2 * kept * d * es + (13 * k + 8) * T, peak_tflops=None)
    if stage == "combine":
        return dict(flops=0.0, bytes=(kept + 2 * T) * d * es + 13 * k * T, peak_tflops=None)
    if stage == "route_rows":
        return dict(flops=0.0, bytes=T * N * 4 + 8 * T, peak_tflops=None)
    return dict(flops=0.0, bytes=0, peak_tflops=None)


def roofline_entry(stage: str, work: dict, ms: float) -> dict:
    sec = ms * 1e-3
    t_mfma = work["flops"] / (work["peak_tflops"] * 1e12) if work["peak_tflops"] else 0.0
    t_hbm = work["bytes"] / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm and work["flops"] > 0:
        bound = "mfma" if work["peak_tflops"] == PEAK_BF16_TFLOPS else "alu"
        achieved, peak, unit = work["flops"] / sec / 1e12, work["peak_tflops"], "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", work["bytes"] / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"kernel": stage, "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
            "algorithmic_flops": work["flops"], "algorithmic_bytes": work["bytes"],
            "mean_ms": round(ms, 5),
            "mfma_frac": round(work["flops"] / sec / 1e12 / PEAK_BF16_TFLOPS, 4)
            if work["flops"] else None}


# stage of the forward call -> (regular expression over the kernel's name in the
# hardware-counter profiles, its source file)
STAGE_KERNEL = {"gemm1_relu": (r"gemm_bf16_\w+<(\d+, \d+, )?true, 1(, false)?>", "gemm.hip"),
                "gemm2": (r"gemm_bf16_\w+<(\d+, \d+, )?false, 0(, false)?>", "gemm.hip"),
                "gemm2_combine": (r"gemm_bf16_\w+<(\d+, \d+, )?false, 2(, false)?>", "gemm.hip"),
                "router": (r"router_\w+(<.*>)?", "router.hip"),
                "dispatch": (r"dispatch_index_kernel", "move.hip"),
                "assign": (r"assign_kernel", "assign.hip"),
                "combine": (r"combine_kernel<.*>", "move.hip")}


_TRAFFIC_LINE = re.compile(
    r"traffic: workload=(?P<workload>\S+) kernel=(?P<kernel>.+?) bytes_per_launch=(?P<bytes_per_launch>\d+)"
    r" source=(?P<source>\S+) source_sha256=(?P<source_sha256>[0-9a-f]+)\s*$")


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed counter profiles (FETCH_SIZE and
    WRITE_SIZE, scaled by a 1 GiB copy), or None when there is no figure for this
    kernel and workload or its source has changed since the counters were taken."""
    if stage not in STAGE_KERNEL:
        return None
    pattern, src = STAGE_KERNEL[stage]
    h = hashlib.sha256()
    for f in (src, "common.hpp"):
        with open(os.path.join(ROOT, "switch_transformer_top_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_bytes.md")):
        with open(path, encoding="utf-8") as fh:
            for line in fh:
                m = _TRAFFIC_LINE.match(line)
                if not m:
                    continue
                kv = m.groupdict()
                k = kv.get("kernel", "")
                if (kv.get("workload") == workload and re.fullmatch(pattern, k)
                        and kv.get("source_sha256") == digest):
                    return float(kv["bytes_per_launch"])
    return None


def cpu_baseline(spec, host, budget_s: float, top_k: int = 1) -> dict:
    """The oracle as it stands on the host cores, over a bounded sample."""
    import oracle
    nt = oracle.threads()
    if spec.N * spec.F * spec.d <= 2e8:
        # the whole workload fits in host memory: run it whole, as often as the budget allows
        xf = S.to_f32(host["x"], spec.act)
        W_in = S.to_f32(host["W_in"], spec.expert)
        W_out = S.to_f32(host["W_out"], spec.expert)
        reps, t0 = 0, time.perf_counter()
        while True:
            if top_k == 1:
                oracle.forward(xf, host["W_r"], host["b_r"], W_in, W_out, spec.c,
                               spec.capacity_override, spec.alpha, nthreads=nt)
            else:
                h = oracle.logits(xf, host["W_r"], host["b_r"], nthreads=nt)
                r = oracle.route_topk(h, top_k, spec.c, spec.capacity_override, spec.alpha,
                                      nthreads=nt)
                oracle.combine_topk(xf, r["expert_idx"], r["gate"], r["drop"], W_in, W_out,
                                    nthreads=nt)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        return {"value": round(spec.T * reps / el, 1), "unit": "tokens/s", "cores": nt,
                "kind": "oracle",
                "sample": f"full {spec.name} workload (T={spec.T}) x {reps} run(s), "
                          f"{el:.1f} s, fp64 C oracle"}
    # large banks: logits and routing of a token prefix, expert FFN of a shorter
    # prefix (per-token costs do not depend on which tokens or experts they are)
    n_r = int(min(spec.T, max(1024, 2e9 // (spec.d * spec.N))))
    xf = S.to_f32(host["x"][:n_r], spec.act)
    t0 = time.perf_counter()
    h = oracle.logits(xf, host["W_r"], host["b_r"], nthreads=nt)
    r = oracle.route_topk(h, top_k, spec.c, spec.capacity_override, spec.alpha, nthreads=nt)
    t_route = time.perf_counter() - t0
    del h
    n, t_ffn = 0, 0.0
    cache = {}
    t1 = time.perf_counter()
    while t_ffn < budget_s and n < n_r:
        for j in range(top_k):   # one expert FFN per choice of the token
            e = int(r["expert_idx"][n, j])
            if e not in cache:
                tg = time.perf_counter()
                cache = {e: (S.to_f32(S.expert_slice(spec, S.TENSOR_WIN, e), spec.expert),
                             S.to_f32(S.expert_slice(spec, S.TENSOR_WOUT, e), spec.expert))}
                t1 += time.perf_counter() - tg   # weight regeneration is not oracle work
            oracle.token_output(xf[n], r["drop"][n, j], r["gate"][n, j], *cache[e])
        n += 1
        t_ffn = time.perf_counter() - t1
    per_token = t_route / n_r + t_ffn / n
    return {"value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": nt,
            "kind": "oracle",
            "sample": f"{spec.name}: logits and routing of the first {n_r} tokens "
                      f"({t_route:.1f} s, {nt} threads) plus the expert FFN of the first {n} "
                      f"tokens ({t_ffn:.1f} s, 1 thread); rate = 1 / per-token time"}


def build_layer(spec, B, torch, dev, top_k: int = 1):
    if spec_id_of(spec) in DEVICE_WEIGHTS:
        host = S.host_inputs(spec, with_experts=False)
        per = spec.N * spec.F * spec.d
        W_in = torch.empty(per, dtype=torch.int16, device=dev)
        W_out = torch.empty(per, dtype=torch.int16, device=dev)
        S.gpu_fill(spec, S.TENSOR_WIN, W_in.data_ptr(), 0, per)
        S.gpu_fill(spec, S.TENSOR_WOUT, W_out.data_ptr(), 0, per)
        W_r = torch.from_numpy(host["W_r"]).to(dev)
        b_r = None if host["b_r"] is None else torch.from_numpy(host["b_r"]).to(dev)
        cfg = B.switch_config(t_max=spec.T, d_model=spec.d, d_ff=spec.F, n_experts=spec.N,
                              capacity_factor=spec.c, capacity_override=0, alpha=spec.alpha,
                              act_dtype=B.SWITCH_BF16, expert_dtype=B.SWITCH_BF16, top_k=top_k)
        return host, B.SwitchLayer(cfg, W_r, b_r, W_in, W_out)
    host = S.host_inputs(spec)
    return host, B.SwitchLayer.from_host(spec, host, device=dev, top_k=top_k)


def spec_id_of(spec) -> int:
    for k, v in S.CONFIGS.items():
        if v == spec:
            return k
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=sorted(S.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--top-k", type=int, default=1, choices=(1, 2),
                    help="experts per token: 1 is the Switch layer (the headline); 2 times the "
                         "top-2 routing variant on the same workload")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (gradients of every input and weight) "
                         "after the forward, and report it beside the forward line's fields")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one by one after writing a 512 MiB buffer (larger than the "
                         "256 MB Infinity Cache), so every step starts with cold caches; 0: skip")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, run one device-to-device copy of 1 GiB "
                         "(reference for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build runs the Switch layer on a single "
              "MI355X and has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from switch_transformer_top_amd import binding as B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    spec = S.CONFIGS[args.config]
    host, layer = build_layer(spec, B, torch, dev, args.top_k)
    workload = spec.name if args.top_k == 1 else f"{spec.name}-top{args.top_k}"
    x = B.to_device(host["x"], dev)
    bufs = layer.alloc(spec.T)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    for _ in range(args.warmup):
        layer.forward(x, spec.T, bufs, stream=sp, with_logits=False)
    torch.cuda.synchronize()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        layer.forward(x, spec.T, bufs, stream=sp, with_logits=False)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(stop) / args.steps

    # cold caches: before each step a 512 MiB write evicts the weights, x and the
    # workspace from L2 and the Infinity Cache; only the step itself is timed
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.cold_steps)]
        for a, b in ev:
            flush.fill_(1)
            a.record(stream)
            layer.forward(x, spec.T, bufs, stream=sp, with_logits=False)
            b.record(stream)
        torch.cuda.synchronize()
        cold_ms = sum(a.elapsed_time(b) for a, b in ev) / args.cold_steps
        cold = {"ms_per_step": round(cold_ms, 5),
                "tokens_per_s": round(spec.T / (cold_ms * 1e-3), 1),
                "steps": args.cold_steps, "flush_bytes": 512 << 20}
        del flush

    # second pass of K steps: the library records HIP events around every kernel
    B.switch_profile_enable(layer.handle, args.steps)
    for _ in range(args.steps):
        layer.forward(x, spec.T, bufs, stream=sp, with_logits=False)
    stage_ms = dict(B.switch_profile_read(layer.handle))
    B.switch_profile_enable(layer.handle, 0)
    torch.cuda.synchronize()

    backward = None
    if args.backward:
        # the training forward: logits for the backward's routing, and the expert
        # outputs kept in its workspace (switch_set_keep_expert_out), timed on its own
        B.switch_set_keep_expert_out(layer.handle, True)
        for _ in range(args.warmup):
            layer.forward(x, spec.T, bufs, stream=sp, with_logits=True)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(args.steps):
            layer.forward(x, spec.T, bufs, stream=sp, with_logits=True)
        f1.record(stream)
        torch.cuda.synchronize()
        train_fwd_ms = f0.elapsed_time(f1) / args.steps
        B.switch_set_keep_expert_out(layer.handle, False)
        gen = torch.Generator(device=dev).manual_seed(1000 + spec.seed)   # seeded dL/dout
        g_out = torch.randn((spec.T, spec.d), device=dev, generator=gen).to(torch.bfloat16)
        g_out = g_out.view(torch.int16)
        grads = layer.alloc_backward(spec.T)
        for _ in range(args.warmup):
            layer.backward(x, spec.T, g_out, 1.0, bufs, grads, stream=sp, reuse_forward=True)
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(args.steps):
            layer.backward(x, spec.T, g_out, 1.0, bufs, grads, stream=sp, reuse_forward=True)
        b1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / args.steps
        B.switch_profile_enable(layer.handle, args.steps)
        for _ in range(args.steps):
            layer.backward(x, spec.T, g_out, 1.0, bufs, grads, stream=sp, reuse_forward=True)
        bwd_stages = dict(B.switch_profile_read(layer.handle))
        B.switch_profile_enable(layer.handle, 0)
        torch.cuda.synchronize()
        bwd_kept = int((B.from_device(bufs["drop_mask"]) == 0).sum())
        # matmul work of the backward: four gradient matmuls over the kept assignments
        # (H and Y come from the training forward's workspace; the weight-gradient K
        # runs over padded rows)
        bwd_flops = 8.0 * bwd_kept * spec.d * spec.F
        backward = {"ms_per_step": round(bwd_ms, 5),
                    "tokens_per_s": round(spec.T / (bwd_ms * 1e-3), 1),
                    "train_forward_ms": round(train_fwd_ms, 5),
                    "fwd_bwd_tokens_per_s": round(spec.T / ((bwd_ms + train_fwd_ms) * 1e-3), 1),
                    "matmul_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
                    "stage_ms": {k: round(v, 5) for k, v in bwd_stages.items()}}

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    drop = B.from_device(bufs["drop_mask"])
    load = B.from_device(bufs["load"])
    kept = int((drop == 0).sum())          # kept assignments (tokens at top-1)
    C = B.switch_capacity(layer.handle, spec.T)
    active = int((np.minimum(load, C) > 0).sum())

    rooflines = {k: roofline_entry(k, stage_work(k, spec, kept, active, args.top_k), v)
                 for k, v in stage_ms.items()
                 if k in ("router", "router_logits", "gemm1_relu", "gemm2", "gemm2_combine",
                          "dispatch", "combine")}
    dominant = max(rooflines, key=lambda k: stage_ms[k])
    for k, r in rooflines.items():
        r["traffic"] = measured_traffic(k, workload)
    gemm_ms = (stage_ms.get("gemm1_relu", 0) + stage_ms.get("gemm2", 0)
               + stage_ms.get("gemm2_combine", 0))
    expert_tflops = 4.0 * kept * spec.d * spec.F / (gemm_ms * 1e-3) / 1e12 if gemm_ms else 0.0

    result = {
        "metric": METRIC,
        "value": round(spec.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.act,
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": workload, "T": spec.T, "d_model": spec.d, "d_ff": spec.F,
                   "n_experts": spec.N, "capacity_factor": spec.c, "capacity": C,
                   "router": "fp32", "experts": spec.expert, "parallelism": "single-gpu"},
        "roofline": rooflines[dominant],
        "cpu_baseline": None,
        "top_k": args.top_k,
        "kept_assignments": kept,
        "dropped_assignments": spec.T * args.top_k - kept,
        "expert_tflops": round(expert_tflops, 2),
        "expert_mfma_frac": round(expert_tflops / PEAK_BF16_TFLOPS, 4),
        "dispatch_hbm_frac": rooflines.get("dispatch", rooflines.get("assign", {})).get("frac"),
        "combine_hbm_frac": rooflines.get("combine", {}).get("frac"),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stage_rooflines": rooflines,
        "wall_s_timed_region": round(wall, 4),
    }
    if cold is not None:
        result["cold_cache"] = cold
    if backward is not None:
        result["backward"] = backward
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, host, args.cpu_budget, args.top_k)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
