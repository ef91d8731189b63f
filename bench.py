#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE FFN layer (Q4_K experts) on one MI355X.

One step = one call of the layer (router, bucketing, staging, gate/up with
SwiGLU, down, combine) on one batch of T tokens already resident in HBM.
The default workload is the Qwen3-30B-A3B-shaped decode layer (H=2048, E=128,
k=8, I=768, T=1); the 2048-token Zipf-routed prefill of the same shape is
measured beside it and reported under "prefill".

Timing: W warmup steps, then K steps captured in one HIP graph and replayed
between two events on the launch stream, with device synchronisation on both
sides. Steps cycle over R replicas of the layer (distinct weights and inputs)
whose weights total >= 1 GB, so the 256 MB Infinity Cache cannot hold the
working set. The dominant kernel (gate_up) is then timed over K more eager
steps with events stamped at its own start and end (hipExtLaunchKernelGGL);
its roofline fraction uses algorithmic bytes (decode: routed gate+up Q4_K
weight bytes) or flops (prefill: 2*T*k*2*H*I) per launch.

Single eager steps (median, 10th / 90th percentile) go under "step_us": "warm" with
only a GPU sleep between steps, "cold" with a 512 MB write between steps (outside
the timed events) that leaves no weight or input in any cache.

The layer inside its block (moe_ffn_forward_block: pre-FFN RMSNorm, the layer, residual
add) is timed the same way on the decode and prefill workloads under "block", with the
time of one per-stage statistics call (moe_ffn_debug_stats) on the last token.

The decode layer with Q8_K-style int8 expert activations (moe_ffn_forward_q8) is timed
the same way under "q8_activations".

The 64-token batch and the 235b-shaped layer are timed as whole steps under "others".
For context, hbm_step.plain_copy_probe times a plain device copy of 7, 14 and 21 MiB
(the decode kernels' weight bytes) the same way.

The CPU baseline is the fp64 oracle as it stands, timed on this host on a
bounded sample of the same workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-FFN tokens/s per layer + HBM GB/s (decode), MFMA TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
REPLICA_BYTES = 1 << 30        # weights cycled per timed loop


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="30b-decode")
    ap.add_argument("--prefill-workload", default="30b-prefill")
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-block", action="store_true", help="skip timing the layer inside its block")
    ap.add_argument("--extra-workloads", default="30b-batch,235b-shape",
                    help="comma-separated workloads whose whole-step time is reported under \"others\" ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--stages", action="store_true", help="also time every stage (eager pass, to stderr)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


class Bench:
    """R replicas of one workload on the GPU, with their outputs preallocated."""

    def __init__(self, wl, replicas: int, seed: int = 1, block: bool = False, q8: bool = False):
        import torch

        import synth
        from tests import parity

        self.wl = wl
        self.block = block
        self.q8 = q8
        self.layers, self.xs, self.outs, self.ws, self.idxs = [], [], [], [], []
        self.host0 = None
        for r in range(replicas):
            log(f"{wl.name}: generating replica {r + 1}/{replicas}")
            inp = synth.make_inputs(wl, seed=seed, replica=r)
            dev = parity.upload(inp)
            layer, _ = parity.make_layer(inp, dev)
            layer.reserve(wl.tokens)
            if block:
                layer.set_norm(torch.from_numpy(synth.gen_norm(seed, r, wl.hidden)), synth.NORM_EPS)
            x = dev["x"]
            for key in ("gate", "up", "down", "router", "bias"):
                dev[key] = None  # the layer owns its copies
            if r == 0:
                self.host0 = inp
            self.layers.append(layer)
            self.xs.append(x)
            self.outs.append(torch.empty_like(x))
            self.ws.append(torch.empty((wl.tokens, wl.top_k), dtype=torch.float32, device=x.device))
            self.idxs.append(torch.empty((wl.tokens, wl.top_k), dtype=torch.int32, device=x.device))
        torch.cuda.synchronize()

    @property
    def R(self):
        return len(self.layers)

    def step(self, i: int) -> None:
        r = i % self.R
        if self.block:
            self.layers[r].forward_block(self.xs[r], self.outs[r], self.ws[r], self.idxs[r])
        elif self.q8:
            self.layers[r].forward_q8(self.xs[r], self.outs[r], self.ws[r], self.idxs[r])
        else:
            self.layers[r].forward(self.xs[r], self.outs[r], self.ws[r], self.idxs[r])

    def routing(self):
        """Per replica: (distinct experts U, max tokens on one expert, rows in GEMM buckets)."""
        import numpy as np
        import torch

        for r in range(self.R):
            self.step(r)
        torch.cuda.synchronize()
        stats = []
        for r in range(self.R):
            idx = self.idxs[r].cpu().numpy()
            cnt = np.bincount(idx.ravel(), minlength=self.wl.experts)
            # rows that take the grouped GEMM: buckets of more than 16 entries
            stats.append((int((cnt > 0).sum()), int(cnt.max()), int(cnt[cnt > 16].sum())))
        return stats

    def timed(self, steps: int, warmup: int, eager: bool) -> float:
        """Milliseconds per step."""
        import torch

        torch.cuda.synchronize()
        if eager:
            for i in range(warmup):
                self.step(i)
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for i in range(steps):
                self.step(i)
            end.record()
            torch.cuda.synchronize()
            return start.elapsed_time(end) / steps
        gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, capture_error_mode="relaxed"):
            for i in range(max(warmup, 1)):
                self.step(i)
        with torch.cuda.graph(gt, capture_error_mode="relaxed"):
            for i in range(steps):
                self.step(i)
        torch.cuda.synchronize()
        gw.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        gt.replay()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        del gw, gt
        return ms

    def per_step(self, n: int, flush_mb: int = 512) -> dict:
        """Median and 10th / 90th percentile of single-step times (us): n eager steps, cycling over the replicas,
        each between two events. "warm": a GPU sleep (no memory traffic) before each step, long enough for the host
        to have queued the step before it starts; "cold": a write of flush_mb MB before each step (outside the
        events), so no weight or input is left in L2 or the Infinity Cache."""
        import numpy as np
        import torch

        flush = torch.empty(flush_mb * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        res = {}
        for mode in ("warm", "cold"):
            for r in range(self.R):
                self.step(r)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for i in range(n):
                if mode == "cold":
                    flush.fill_(float(i))
                else:
                    torch.cuda._sleep(200_000)
                ev[i][0].record()
                self.step(i)
                ev[i][1].record()
            torch.cuda.synchronize()
            us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
            res[mode] = {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
                         "p90": round(float(np.percentile(us, 90)), 2), "steps": n}
        del flush
        res["flush_mb"] = flush_mb
        log(f"{self.wl.name}: single-step us {res}")
        return res

    def stage_times(self, steps: int, stages) -> dict:
        """{stage: [(replica, total ms, launches)]} from kernel-stamped events over `steps` eager steps."""
        import torch

        import quantized_moe_wave_amd as q

        for layer in self.layers:
            q.moe_ffn_profile(layer.handle, stages)
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        res = {s: [] for s in stages}
        for r, layer in enumerate(self.layers):
            got = q.moe_ffn_profile_read(layer.handle)
            q.moe_ffn_profile(layer.handle, [])
            for s in stages:
                res[s].append((r, got[s][0], got[s][1]))
        return res

    def close(self):
        for layer in self.layers:
            layer.close()
        self.layers = []


def measured_traffic(kernel: str):
    """HBM bytes per dispatch of `kernel` from profiles/hbm_traffic.md (rocprofv3 FETCH_SIZE / WRITE_SIZE,
    scaled by the plain-copy calibration), or None if not measured or if the kernel's sources changed since."""
    import hashlib
    import re

    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    k = data["kernels"].get(kernel)
    if k is None:
        return None
    h = hashlib.sha256()
    for f in k["files"]:
        h.update(open(os.path.join(here, "quantized_moe_wave_amd", "csrc", f), "rb").read())
    if h.hexdigest()[:16] != k["source_hash"]:
        return None
    return int(round((k["fetch_kib"] * data["fetch_factor"] + k["write_kib"] * data["write_factor"]) * 1024))


def replicas_for(wl) -> int:
    layer_bytes = wl.experts * wl.expert_bytes + wl.experts * wl.hidden * 4
    return max(1, math.ceil(REPLICA_BYTES / layer_bytes))


def gate_up_bytes_per_expert(wl) -> int:
    return 2 * wl.hidden * wl.inter * 144 // 256


def measure(wl, steps: int, warmup: int, eager: bool, bound: str, want_stages: bool):
    b = Bench(wl, replicas_for(wl))
    try:
        stats = b.routing()
        log(f"{wl.name}: routing per replica (distinct experts, max tokens/expert) = {stats}")
        ms = b.timed(steps, warmup, eager)
        log(f"{wl.name}: {ms * 1e3:.2f} us/step over {steps} steps ({'eager' if eager else 'graph'})")
        T, k, H, I = wl.tokens, wl.top_k, wl.hidden, wl.inter
        if bound == "hbm":
            # decode: the gate/up kernel; routed gate+up weight bytes of each launch
            # (T <= 4: the per-pair decode kernel, else the 16-row grouped GEMM)
            stage = "gate_up"
            kname = "gateup_pair_kernel" if T <= 4 else "expert_gemm_kernel<gate_up, 16-row tiles>"
            prof = b.stage_times(steps, [stage])[stage]
            total_ms = sum(p[1] for p in prof)
            launches = sum(p[2] for p in prof)
            if launches == 0 or total_ms <= 0:
                raise RuntimeError(f"{wl.name}: no {stage} launches were timed")
            alg = sum(stats[r][0] * gate_up_bytes_per_expert(wl) * nl for r, _, nl in prof)
            achieved = alg / (total_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(kname) if T <= 4 else None,
                    "kernel": f"{kname} ({stage})", "avg_us": round(total_ms / launches * 1e3, 3),
                    "algorithmic_bytes_per_launch": int(round(alg / launches))}
        else:
            # prefill: the gate/up grouped GEMM (its 8-wave launch plus the 4-wave launch that runs the split
            # last-round tiles, when there is one); 2 * rows * 2I * H flops per step
            import quantized_moe_wave_amd as q

            stage = "gate_up_big"
            tail = "gate_up_tail" if "gate_up_tail" in q.moe_ffn_stage_names() else None
            both = b.stage_times(steps, [stage] + ([tail] if tail else []))
            prof = [(r, ms + (both[tail][i][1] if tail else 0.0), nl) for i, (r, ms, nl) in enumerate(both[stage])]
            total_ms = sum(p[1] for p in prof)
            launches = sum(p[2] for p in prof)
            if launches == 0 or total_ms <= 0:
                raise RuntimeError(f"{wl.name}: no {stage} launches were timed")
            flops = sum(2.0 * stats[r][2] * 2 * I * H * nl for r, _, nl in prof)
            achieved = flops / (total_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                    "traffic": measured_traffic("expert_gemm_kernel<gate_up, 64-row tiles>"),
                    "kernel": "expert_gemm_kernel<gate_up, 64-row tiles> (gate_up_big + gate_up_tail)",
                    "avg_us": round(total_ms / launches * 1e3, 3)}
        avg_us = total_ms / launches * 1e3
        log(f"{wl.name}: {stage} avg {avg_us:.2f} us/launch -> {roof['achieved']} {roof['unit']}")
        if want_stages:
            import quantized_moe_wave_amd as q

            allp = b.stage_times(steps, q.moe_ffn_stage_names())
            for s, lst in allp.items():
                tm = sum(p[1] for p in lst)
                n = sum(p[2] for p in lst)
                log(f"{wl.name}: stage {s:8s} {tm / max(n, 1) * 1e3:9.2f} us avg over {n} launches")
        U = sum(st[0] for st in stats) / len(stats)
        roof_steps = b.per_step(max(20, min(steps, 200)))
        return b, ms, stats, roof, U, roof_steps
    except Exception:
        b.close()
        raise


def measure_step(wl, steps: int, eager: bool, want_stages: bool = False) -> dict:
    """Whole-step time of one more workload: tokens/s and the step's routed-expert bytes and algorithmic flops
    against the HBM and MFMA peaks."""
    import torch

    b = Bench(wl, replicas_for(wl))
    try:
        stats = b.routing()
        ms = b.timed(steps, max(3, steps // 10), eager)
        if want_stages:
            import quantized_moe_wave_amd as q

            for st, lst in b.stage_times(steps, q.moe_ffn_stage_names()).items():
                n = sum(p[2] for p in lst)
                if n:
                    log(f"{wl.name}: stage {st:12s} {sum(p[1] for p in lst) / n * 1e3:9.2f} us avg over {n} launches")
    finally:
        b.close()
        del b
        torch.cuda.empty_cache()
    log(f"{wl.name}: {ms * 1e3:.2f} us/step over {steps} steps; routing per replica {stats}")
    U = sum(st[0] for st in stats) / len(stats)
    T, k, H, I, E = wl.tokens, wl.top_k, wl.hidden, wl.inter, wl.experts
    step_bytes = U * wl.expert_bytes
    flops = 2.0 * T * k * 3 * H * I + 2.0 * T * E * H
    sec = ms * 1e-3
    return {"workload": wl.name, "tokens": T, "steps": steps, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(T / sec, 1), "distinct_experts": U,
            "max_tokens_per_expert": max(st[1] for st in stats),
            "hbm_step": {"routed_expert_bytes": int(step_bytes), "achieved_gbs": round(step_bytes / sec / 1e9, 1),
                         "frac": round(step_bytes / sec / 1e9 / HBM_PEAK_GBS, 4)},
            "mfma_step": {"algorithmic_tflops": round(flops / sec / 1e12, 2),
                          "frac": round(flops / sec / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}}


def measure_block(wl, steps: int, eager: bool) -> dict:
    """The layer inside its block (moe_ffn_forward_block: RMSNorm, the layer, residual add), timed like the main
    step, with the norm kernel's own time from kernel-stamped events."""
    import torch

    import quantized_moe_wave_amd as q

    b = Bench(wl, replicas_for(wl), block=True)
    try:
        ms = b.timed(steps, max(3, steps // 10), eager)
        st = b.stage_times(steps, ["norm"])["norm"]
        n = sum(p[2] for p in st)
        norm_us = sum(p[1] for p in st) / max(n, 1) * 1e3
        # the per-stage statistics of the last token after a block step (the traced path's summary)
        b.step(0)
        stats = torch.empty((4, 7), dtype=torch.float64, device="cuda")
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(200_000)
        a.record()
        for _ in range(50):
            q.moe_ffn_debug_stats(b.layers[0].handle, wl.tokens - 1, b.outs[0], b.ws[0], stats)
        e.record()
        torch.cuda.synchronize()
        stats_us = a.elapsed_time(e) / 50 * 1e3
    finally:
        b.close()
        del b
        torch.cuda.empty_cache()
    log(f"{wl.name} block: {ms * 1e3:.2f} us/step, norm kernel {norm_us:.2f} us, stage statistics {stats_us:.2f} us")
    return {"workload": wl.name, "tokens": wl.tokens, "steps": steps, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1), "norm_kernel_us": round(norm_us, 3),
            "stage_stats_us": round(stats_us, 2)}


def measure_q8(wl, steps: int, eager: bool) -> dict:
    """The layer with Q8_K-style int8 expert activations (moe_ffn_forward_q8, decode path), timed like the main
    step."""
    import torch

    b = Bench(wl, replicas_for(wl), q8=True)
    try:
        ms = b.timed(steps, max(3, steps // 10), eager)
    finally:
        b.close()
        del b
        torch.cuda.empty_cache()
    log(f"{wl.name} q8 activations: {ms * 1e3:.2f} us/step")
    return {"workload": wl.name, "tokens": wl.tokens, "steps": steps, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1)}


def cpu_baseline(inp, seconds: float):
    """The oracle on T=1 forwards of replica 0's weights, one token per call, for ~seconds."""
    import numpy as np

    import oracle
    import synth

    cores = oracle.set_threads(len(os.sched_getaffinity(0)))
    wl = inp.wl
    n, t0 = 0, time.perf_counter()
    while True:
        x = synth.gen_x(99, n, 1, wl.hidden)
        oracle.forward(x, inp.router, inp.bias, inp.gate, inp.up, inp.down, wl.top_k)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds and n >= 3:
            break
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} single-token forwards of the {wl.name} layer (replica 0 weights), {el:.1f} s"}


def copy_probe(sizes_mb=(7, 14, 21), steps: int = 200) -> dict:
    """Context for the decode roofline: a plain device copy (torch) of the decode kernels' byte counts, timed like a
    step (one HIP graph of `steps` copies cycling over >= 1 GB of sources, so the caches are cold)."""
    import torch

    out = {}
    for mb in sizes_mb:
        n = mb * (1 << 20) // 4
        R = max(4, REPLICA_BYTES // (n * 4))
        src = [torch.randn(n, device="cuda") for _ in range(R)]
        dst = [torch.empty(n, device="cuda") for _ in range(R)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                dst[i % R].copy_(src[i % R])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        out[f"{mb}MiB"] = {"us": round(us, 2), "read_GBs": round(n * 4 / us / 1e3, 1)}
        del src, dst, g
        torch.cuda.empty_cache()
    log(f"plain copy probe: {out}")
    return out


def copy_calibration(mb: int) -> None:
    import torch

    n = mb * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.add(a, 0.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))


def main() -> int:
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and timed on a single MI355X "
              "(run with --gpus 1).", file=sys.stderr)
        return 2
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)
        return 0
    import torch

    import synth

    from quantized_moe_wave_amd.build import LIB

    if not os.path.exists(LIB):
        import __graft_entry__

        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    wl = synth.WORKLOADS[args.workload]
    b, ms, stats, roof, U, dist = measure(wl, args.steps, args.warmup, args.eager, "hbm", args.stages)
    host0 = b.host0
    b.close()
    del b
    torch.cuda.empty_cache()
    value = wl.tokens / (ms * 1e-3)
    step_bytes = U * wl.expert_bytes
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "hidden": wl.hidden, "experts": wl.experts, "top_k": wl.top_k,
                   "moe_intermediate": wl.inter, "tokens": wl.tokens, "replicas": replicas_for(wl),
                   "timing": "eager" if args.eager else "hip-graph"},
        "hbm_step": {"routed_expert_bytes": int(step_bytes), "achieved": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                     "unit": "GB/s", "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "distinct_experts": U},
        "roofline": roof,
        "step_us": dist,
    }
    if not args.no_prefill:
        pw = synth.WORKLOADS[args.prefill_workload]
        pb, pms, pstats, proof, pU, pdist = measure(pw, args.prefill_steps, max(3, args.prefill_steps // 10), args.eager,
                                             "mfma", args.stages)
        pb.close()
        del pb
        torch.cuda.empty_cache()
        flops = 2.0 * pw.tokens * pw.top_k * 3 * pw.hidden * pw.inter + 2.0 * pw.tokens * pw.experts * pw.hidden
        line["prefill"] = {
            "workload": pw.name, "tokens": pw.tokens, "steps": args.prefill_steps, "ms_per_step": round(pms, 4),
            "tokens_per_s": round(pw.tokens / (pms * 1e-3), 1),
            "tflops": round(flops / (pms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(flops / (pms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "distinct_experts": pU, "max_tokens_per_expert": max(st[1] for st in pstats),
            "gemm_rows": sum(st[2] for st in pstats) / len(pstats), "roofline": proof, "step_us": pdist,
        }
    if not args.no_block:
        line["block"] = [measure_block(wl, args.steps, args.eager)]
        if not args.no_prefill:
            line["block"].append(measure_block(synth.WORKLOADS[args.prefill_workload], args.prefill_steps, args.eager))
    if wl.tokens <= 4:
        line["q8_activations"] = measure_q8(wl, args.steps, args.eager)
    line["hbm_step"]["plain_copy_probe"] = copy_probe()
    extras = [w for w in args.extra_workloads.split(",") if w]
    if extras:
        line["others"] = [measure_step(synth.WORKLOADS[w], args.extra_steps, args.eager, args.stages) for w in extras]
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {wl.name} for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(host0, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
