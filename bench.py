"""Benchmark of the Switch FFN layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 5] [--no-cpu-baseline]

One step = one switch_forward call over the whole workload (router, softmax and
top-1, capacity assignment, load-balancing loss, dispatch, both expert matmuls,
combine) on seeded synthetic inputs already resident in HBM.  The default
workload is the largest single-GPU one: one GPU's share of a 2048-expert
Switch layer, T=131072 tokens, d_model=2048, d_ff=6144, capacity factor 1.0
(about 103 GB of bf16 expert weights).

Timing: W untimed steps, then K steps each timed with HIP events on the
library's stream after a 512 MiB read that evicts L2 and the Infinity Cache
(cold caches, and no dirty lines left to write back); the value is T / the
median step time.  The same K steps after a 512 MiB write each are reported
beside it.  Then K warm steps, a
profiled pass whose per-kernel event means give each kernel's roofline, a
pass of the unfused path that times the stand-alone combine, the attainable
peaks of the box (an MFMA loop and HBM streams), and the CPU oracle on the
host cores.  Prints one JSON line.
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
    if stage == "ffn_fused":
        # both matmuls with the combine, H on chip: the weights of the experts in
        # use, the kept rows of x in, the residual rows in and the outputs out
        return dict(flops=4.0 * kept * d * F,
                    bytes=2 * active_experts * d * F * es + 3 * kept * d * es + 8 * kept,
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
STAGE_KERNEL = {"gemm1_relu": (r"gemm_bf16_\w+<(\d+, \d+, )?true, 1(, (false|true)(, \d+)?)?>",
                               "gemm.hip"),
                "gemm2": (r"gemm_bf16_\w+<(\d+, \d+, )?false, 0(, (false|true)(, \d+)?)?>",
                          "gemm.hip"),
                "gemm2_combine": (r"gemm_bf16_\w+<(\d+, \d+, )?false, 2(, (false|true)(, \d+)?)?>",
                                  "gemm.hip"),
                "router": (r"router_(small|tok)_kernel(<.*>)?", "router.hip"),
                "router_logits": (r"router_gemm_dma_kernel", "router.hip"),
                "route_rows": (r"route_rows\w*(<.*>)?", "router.hip"),
                "route_scan": (r"route_scan_kernel", "assign.hip"),
                "ffn_fused": (r"ffn_fused_kernel(<.*>)?", "ffn.hip"),
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
    for f in (src, "common.hpp", "epilogue.hpp"):
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


def host_info() -> dict:
    """The host the oracle runs on: logical CPUs, the process's affinity mask, CPU model."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model}


def _oracle_whole(oracle, spec, host, top_k, nt, budget_s):
    """Whole-workload oracle runs with nt threads, as often as the budget allows."""
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
            return reps, el


def _oracle_prefix_single(oracle, spec, host, top_k, xf, r, tk, jk, ek, budget_s):
    """Seconds per token of the prefix sample on one thread: the routing of up to
    256 tokens and the FFN of the first experts' assignments, each within the budget."""
    n1 = min(len(xf), 256)
    t0 = time.perf_counter()
    h = oracle.logits(xf[:n1], host["W_r"], host["b_r"], nthreads=1)
    oracle.route_topk(h, top_k, spec.c, spec.capacity_override, spec.alpha, nthreads=1)
    t_route = (time.perf_counter() - t0) / n1
    n_ffn, t_ffn, i = 0, 0.0, 0
    while i < len(tk) and t_ffn < budget_s:
        j = i + 1
        while j < len(tk) and ek[j] == ek[i] and j - i < 8:
            j += 1
        e = int(ek[i])
        W_in = S.to_f32(S.expert_slice(spec, S.TENSOR_WIN, e), spec.expert)[None]
        W_out = S.to_f32(S.expert_slice(spec, S.TENSOR_WOUT, e), spec.expert)[None]
        t1 = time.perf_counter()
        oracle.combine(xf[tk[i:j]], np.zeros(j - i, np.int32), r["gate"][tk[i:j], jk[i:j]],
                       np.zeros(j - i, np.uint8), W_in, W_out, nthreads=1)
        t_ffn += time.perf_counter() - t1
        n_ffn += j - i
        i = j
    return t_route + top_k * t_ffn / max(1, n_ffn)


def cpu_baseline(spec, host, budget_s: float, top_k: int = 1) -> dict:
    """The oracle as it stands on every host core the process may use, over a bounded
    sample; one thread as well for the workloads the oracle runs whole."""
    import oracle
    nt = oracle.threads()
    info = host_info()
    if spec.N * spec.F * spec.d <= 2e8:
        # the whole workload fits in host memory: run it whole, as often as the budget allows
        reps, el = _oracle_whole(oracle, spec, host, top_k, nt, budget_s)
        reps1, el1 = _oracle_whole(oracle, spec, host, top_k, 1, budget_s / 2)
        return {"value": round(spec.T * reps / el, 1), "unit": "tokens/s", "cores": nt,
                "kind": "oracle",
                "sample": f"full {spec.name} workload (T={spec.T}) x {reps} run(s), "
                          f"{el:.1f} s, fp64 C oracle, {nt} threads",
                "single_thread_value": round(spec.T * reps1 / el1, 1), **info}
    # large banks: logits and routing of a token prefix, then the expert FFN of
    # that prefix's kept assignments in batches of at least `nt` of them: the
    # assignments of consecutive experts (in expert order) share a bank of those
    # experts' weights, regenerated outside the timing, and the oracle runs
    # OpenMP over the batch.  Per-token costs do not depend on which tokens or
    # experts they are.
    n_r = int(min(spec.T, max(2048, 4e9 // (spec.d * spec.N))))
    xf = S.to_f32(host["x"][:n_r], spec.act)
    t0 = time.perf_counter()
    h = oracle.logits(xf, host["W_r"], host["b_r"], nthreads=nt)
    r = oracle.route_topk(h, top_k, spec.c, spec.capacity_override, spec.alpha, nthreads=nt)
    t_route = time.perf_counter() - t0
    del h
    tk, jk = np.nonzero(r["drop"] == 0)
    ek = r["expert_idx"][tk, jk]
    order = np.argsort(ek, kind="stable")
    tk, jk, ek = tk[order], jk[order], ek[order]
    n_ffn, t_ffn, n_exp, i = 0, 0.0, 0, 0
    wall0 = time.perf_counter()
    while i < len(tk) and t_ffn < budget_s and time.perf_counter() - wall0 < 4 * budget_s:
        j = min(len(tk), i + nt)
        while j < len(tk) and ek[j] == ek[j - 1]:
            j += 1   # an expert's assignments stay in one batch
        experts, slot = np.unique(ek[i:j], return_inverse=True)
        W_in = np.stack([S.to_f32(S.expert_slice(spec, S.TENSOR_WIN, int(e)), spec.expert)
                         for e in experts])
        W_out = np.stack([S.to_f32(S.expert_slice(spec, S.TENSOR_WOUT, int(e)), spec.expert)
                          for e in experts])
        t1 = time.perf_counter()
        oracle.combine(xf[tk[i:j]], slot.astype(np.int32), r["gate"][tk[i:j], jk[i:j]],
                       np.zeros(j - i, np.uint8), W_in, W_out, nthreads=nt)
        t_ffn += time.perf_counter() - t1
        n_ffn += j - i
        n_exp += len(experts)
        i = j
        del W_in, W_out
    per_token = t_route / n_r + top_k * t_ffn / n_ffn
    single = None
    if nt > 1:
        single = round(1.0 / _oracle_prefix_single(oracle, spec, host, top_k, xf, r, tk, jk, ek,
                                                   budget_s / 4), 2)
    return {"value": round(1.0 / per_token, 2), "unit": "tokens/s", "cores": nt,
            "single_thread_value": single,
            "kind": "oracle",
            "sample": f"{spec.name}: logits and routing of the first {n_r} tokens "
                      f"({t_route:.1f} s) plus the expert FFN of {n_ffn} of their kept "
                      f"assignments over {n_exp} expert(s) ({t_ffn:.1f} s), {nt} threads; "
                      f"rate = 1 / (routing time per token + k x FFN time per assignment)",
            **info}


# ------------------------------------------------------------------ attainable peaks

class CacheEvict:
    """Reads a 512 MiB buffer that is never written (twice the Infinity Cache,
    64x an XCD's L2) with the streaming read probe: what the next step reads
    then comes from HBM, and no dirty line is left to be written back."""

    def __init__(self, torch, dev, stream):
        import ctypes
        from switch_transformer_top_amd import build as lb
        self.L = ctypes.CDLL(lb.PEAKS_LIB)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        self.L.peak_hbm_read.argtypes = [vp, i64, vp, vp]
        self.L.peak_stream_blocks.restype = ctypes.c_int
        self.nbytes = 512 << 20
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=dev)
        self.sink = torch.empty(max(1, self.L.peak_stream_blocks()), dtype=torch.int32,
                                device=dev)
        self.stream = stream

    def __call__(self):
        if self.L.peak_hbm_read(self.buf.data_ptr(), self.nbytes, self.sink.data_ptr(),
                                self.stream) != 0:
            raise RuntimeError("cache-evicting read failed to launch")


def attainable_peaks(torch, dev, stream) -> dict:
    """What the box reaches with plain probes (best of five launches each): bf16 MFMA
    (v_mfma_f32_32x32x16_bf16 loop, register operands), and HBM read, write and copy
    streams over 4 GiB (16x the Infinity Cache)."""
    import ctypes
    from switch_transformer_top_amd import build as lb
    L = ctypes.CDLL(lb.PEAKS_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.peak_mfma_bf16.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    L.peak_hbm_read.argtypes = [vp, i64, vp, vp]
    L.peak_hbm_write.argtypes = [vp, i64, vp]
    L.peak_hbm_copy.argtypes = [vp, vp, i64, vp]
    L.peak_stream_blocks.restype = ctypes.c_int
    props = torch.cuda.get_device_properties(dev)
    blocks, iters = 8 * props.multi_processor_count, 4000
    sink = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rsink = torch.empty(max(1, L.peak_stream_blocks()), dtype=torch.int32, device=dev)

    def best(launch, reps=5):
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if launch() != 0:
                raise RuntimeError("peak probe launch failed")
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    half = nbytes // 2
    t_mfma = best(lambda: L.peak_mfma_bf16(sink.data_ptr(), blocks, iters, stream))
    t_write = best(lambda: L.peak_hbm_write(buf.data_ptr(), nbytes, stream))
    t_read = best(lambda: L.peak_hbm_read(buf.data_ptr(), nbytes, rsink.data_ptr(), stream))
    t_copy = best(lambda: L.peak_hbm_copy(buf.data_ptr(), buf.data_ptr() + half, half, stream))
    del buf
    flops = blocks * 4.0 * iters * 4 * 32768
    return {"mfma_bf16_tflops": round(flops / (t_mfma * 1e-3) / 1e12, 1),
            "hbm_read_gbs": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "hbm_write_gbs": round(nbytes / (t_write * 1e-3) / 1e9, 1),
            "hbm_copy_gbs": round(2 * half / (t_copy * 1e-3) / 1e9, 1),
            "probe": "best of 5 launches; MFMA: 8 blocks of 4 waves per CU, 4 independent "
                     "32x32x16 bf16 chains per wave; HBM: 4 GiB streams, each XCD over its own "
                     "contiguous eighth (copy: 2 GiB read + 2 GiB written, counted as 4 GiB)"}


# stages whose HBM traffic is almost all reads (weights, tokens, logits): their
# attainable reference is the read stream; the movers' is the copy stream
READ_STAGES = ("router", "router_logits", "route_rows", "gemm1_relu", "gemm2", "gemm2_combine",
               "ffn_fused")


def with_attainable(entry: dict, peaks) -> dict:
    """Add the fraction of the measured attainable peak of the entry's bound."""
    if not peaks or entry is None:
        return entry
    if entry["bound"] == "hbm":
        ref = "hbm_read_gbs" if entry["kernel"] in READ_STAGES else "hbm_copy_gbs"
        entry["attainable_ref"] = ref
        entry["frac_attainable"] = round(entry["achieved"] / peaks[ref], 4)
    elif entry["bound"] == "mfma":
        entry["attainable_ref"] = "mfma_bf16_tflops"
        entry["frac_attainable"] = round(entry["achieved"] / peaks["mfma_bf16_tflops"], 4)
    return entry


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


def load_summary(load, C: int) -> dict:
    """The realised per-expert loads (assignments before the capacity cut)."""
    load = np.asarray(load, dtype=np.int64)
    return {"min": int(load.min()), "p50": float(np.percentile(load, 50)),
            "p99": float(np.percentile(load, 99)), "max": int(load.max()),
            "empty_experts": int((load == 0).sum()), "over_capacity": int((load > C).sum()),
            "top8": [int(v) for v in np.sort(load)[::-1][:8]]}


def median(v):
    return float(np.median(np.asarray(v, dtype=np.float64)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=sorted(S.CONFIGS),
                    help="workload (1-5); 5, the 2048-expert share, is the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak probes (MFMA loop, HBM streams)")
    ap.add_argument("--top-k", type=int, default=1, choices=(1, 2),
                    help="experts per token: 1 is the Switch layer (the headline); 2 times the "
                         "top-2 routing variant on the same workload")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (gradients of every input and weight) "
                         "after the forward, and report it beside the forward line's fields")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, run one device-to-device copy of 1 GiB "
                         "(reference for hardware byte counters)")
    ap.add_argument("--ffn", choices=("auto", "fused", "unfused"), default="auto",
                    help="expert FFN variant: the library's choice (default), the fused kernel "
                         "(H on chip), or the two matmul launches")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run only W warm-up and this many plain steps (for rocprofv3)")
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
    B.switch_set_ffn_mode(layer.handle, {"auto": B.SWITCH_FFN_AUTO, "fused": B.SWITCH_FFN_FUSED,
                                         "unfused": B.SWITCH_FFN_UNFUSED}[args.ffn])

    def step():
        layer.forward(x, spec.T, bufs, stream=sp, with_logits=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        if args.calibrate_copy:
            a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            torch.cuda.synchronize()
            b.copy_(a)
            torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": workload}), flush=True)
        return

    # timed region: K steps, each after a 512 MiB read that evicts the weights, x
    # and the workspace from L2 and the Infinity Cache (a read leaves no dirty
    # lines whose write-back would land inside the step); only the step is timed
    evict = CacheEvict(torch, dev, sp)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for a, b in ev:
        evict()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    cold = [a.elapsed_time(b) for a, b in ev]
    del evict

    # the same K steps, each after a 512 MiB write instead (the eviction the
    # measurement plan names; the write-back of its dirty lines lands inside the
    # step), reported beside the value
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for a, b in ev:
        flush.fill_(1)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    cold_write = [a.elapsed_time(b) for a, b in ev]
    del flush

    # warm: the same K steps back to back (weights and x may stay in the caches, as
    # between the layers of one model's forward), each timed alone
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) for a, b in ev]

    # profiled pass: the library records HIP events on the dispatches of every kernel
    B.switch_profile_enable(layer.handle, args.steps)
    for _ in range(args.steps):
        step()
    stage_ms = dict(B.switch_profile_read(layer.handle))
    B.switch_profile_enable(layer.handle, 0)
    torch.cuda.synchronize()

    # the stand-alone combine (the separate pass of the unfused path, which the
    # debug entry point runs after storing the expert outputs) timed the same way
    mover_ms = {}
    if "combine" not in stage_ms and spec.act == "bf16":
        Cb = max(0, min(B.switch_capacity(layer.handle, spec.T), spec.T))
        eo = torch.empty((spec.N, Cb, spec.d), dtype=torch.int16, device=dev)
        n_dbg = max(1, min(args.steps, 5))
        layer.forward(x, spec.T, bufs, stream=sp, with_logits=False, expert_out=eo)
        B.switch_profile_enable(layer.handle, n_dbg)
        for _ in range(n_dbg):
            layer.forward(x, spec.T, bufs, stream=sp, with_logits=False, expert_out=eo)
        mover_ms = dict(B.switch_profile_read(layer.handle))
        B.switch_profile_enable(layer.handle, 0)
        torch.cuda.synchronize()
        del eo
        step()   # leave the default path's outputs in bufs
        torch.cuda.synchronize()

    backward = None
    if args.backward:
        backward = time_backward(args, B, torch, dev, spec, layer, x, bufs, sp)

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    peaks = None if args.no_peaks else attainable_peaks(torch, dev, sp)

    drop = B.from_device(bufs["drop_mask"])
    load = B.from_device(bufs["load"])
    kept = int((drop == 0).sum())          # kept assignments (tokens at top-1)
    C = B.switch_capacity(layer.handle, spec.T)
    active = int((np.minimum(load, C) > 0).sum())

    def entry(k, ms):
        e = roofline_entry(k, stage_work(k, spec, kept, active, args.top_k), ms)
        e["traffic"] = measured_traffic(k, workload)
        return with_attainable(e, peaks)

    rooflines = {k: entry(k, v) for k, v in stage_ms.items()
                 if k in ("router", "router_logits", "route_rows", "gemm1_relu", "gemm2",
                          "gemm2_combine", "ffn_fused", "dispatch", "assign", "combine")}
    dominant = max(rooflines, key=lambda k: stage_ms[k])
    gemm_ms = (stage_ms.get("gemm1_relu", 0) + stage_ms.get("gemm2", 0)
               + stage_ms.get("gemm2_combine", 0) + stage_ms.get("ffn_fused", 0))
    expert_tflops = 4.0 * kept * spec.d * spec.F / (gemm_ms * 1e-3) / 1e12 if gemm_ms else 0.0
    slot_stage = "dispatch" if "dispatch" in rooflines else "assign"
    combine_entry = rooflines.get("combine")
    if combine_entry is None and "combine" in mover_ms:
        combine_entry = entry("combine", mover_ms["combine"])
        combine_entry["path"] = ("stand-alone combine pass of the unfused path (expert output "
                                 "stored, then combined); the default top-1 path combines in "
                                 "the second matmul's epilogue")

    cold_ms = median(cold)
    warm_ms = median(warm)
    result = {
        "metric": METRIC,
        "value": round(spec.T / (cold_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.act,
        "data": "synthetic (seeded counter-based generator; random-init weights)",
        "config": {"workload": workload, "T": spec.T, "d_model": spec.d, "d_ff": spec.F,
                   "n_experts": spec.N, "capacity_factor": spec.c, "capacity": C,
                   "router": "fp32", "experts": spec.expert, "parallelism": "single-gpu",
                   "ffn": "fused" if "ffn_fused" in stage_ms else "two launches",
                   "timing": "median of K steps, each after a 512 MiB cache-evicting read "
                             "(cold caches)"},
        "roofline": rooflines[dominant],
        "cpu_baseline": None,
        "top_k": args.top_k,
        "kept_assignments": kept,
        "dropped_assignments": spec.T * args.top_k - kept,
        "kept_tokens_per_s": round(kept / args.top_k / (cold_ms * 1e-3), 1),
        "warm": {"ms_per_step": round(warm_ms, 5),
                 "tokens_per_s": round(spec.T / (warm_ms * 1e-3), 1)},
        "step_ms_cold": {"min": round(min(cold), 5), "max": round(max(cold), 5)},
        "step_ms_cold_write_evict": {"median": round(median(cold_write), 5),
                                     "tokens_per_s": round(spec.T / (median(cold_write) * 1e-3), 1)},
        "loads": load_summary(load, C),
        "expert_tflops": round(expert_tflops, 2),
        "expert_mfma_frac": round(expert_tflops / PEAK_BF16_TFLOPS, 4),
        "dispatch_hbm_frac": rooflines.get(slot_stage, {}).get("frac"),
        "combine_hbm_frac": combine_entry.get("frac") if combine_entry else None,
        "dispatch": rooflines.get(slot_stage),
        "combine": combine_entry,
        "gather_bytes": kept * spec.d * (2 if spec.act == "bf16" else 4),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stage_ms_sum": round(sum(stage_ms.values()), 5),
        "stage_rooflines": rooflines,
        "attainable": peaks,
        "wall_s_timed_region": round(wall, 4),
    }
    if peaks:
        result["expert_mfma_frac_attainable"] = round(expert_tflops / peaks["mfma_bf16_tflops"], 4)
    if backward is not None:
        result["backward"] = backward
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, host, args.cpu_budget, args.top_k)
    print(json.dumps(result), flush=True)


def time_backward(args, B, torch, dev, spec, layer, x, bufs, sp) -> dict:
    """Training forward (logits and expert outputs kept) and the backward pass, warm."""
    stream = torch.cuda.current_stream(dev)
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
    return {"ms_per_step": round(bwd_ms, 5),
            "tokens_per_s": round(spec.T / (bwd_ms * 1e-3), 1),
            "train_forward_ms": round(train_fwd_ms, 5),
            "fwd_bwd_tokens_per_s": round(spec.T / ((bwd_ms + train_fwd_ms) * 1e-3), 1),
            "matmul_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
            "stage_ms": {k: round(v, 5) for k, v in bwd_stages.items()}}


if __name__ == "__main__":
    main()
