#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE FFN layer (Q4_K experts) on one MI355X.

One step = one call of the layer (router, bucketing, staging, gate/up with
SwiGLU, down, combine) on one batch of T tokens already resident in HBM.
The default workload is the Qwen3-30B-A3B-shaped decode layer (H=2048, E=128,
k=8, I=768, T=1); the 2048-token Zipf-routed prefill of the same shape is
measured beside it and reported under "prefill".

Timing: W warmup steps, then K steps captured in one HIP graph and replayed
between two events on the launch stream, with device synchronisation on both
sides. Steps cycle over R replicas of the layer (distinct weights) whose
weights total >= 1 GB, and for T <= 64 over a pool of P = 64 distinct input
batches per replica, so consecutive steps route to different experts: over
the timed loop the experts touched total far more than the 256 MB Infinity
Cache (the JSON line states the union). The dominant kernel is then timed
over K more eager steps with events stamped at its own start and end
(hipExtLaunchKernelGGL); its roofline fraction uses algorithmic bytes (the
routed gate+up Q4_K weight bytes of its launch) or flops (2 * rows * 2I * H
for the 64-row grouped GEMM) per launch.

Single eager steps (median, 10th / 90th percentile) go under "step_us": "warm" with
only a GPU sleep between steps, "cold" with a 512 MB write between steps (outside
the timed events) that leaves no weight or input in any cache.

The layer inside its block (moe_ffn_forward_block: pre-FFN RMSNorm, the layer, residual
add) is timed the same way on the decode and prefill workloads under "block", with the
time of one per-stage statistics call (moe_ffn_debug_stats) on the last token.

The layer with Q8_K-style int8 expert activations (moe_ffn_forward_q8) is timed the
same way under "q8_activations": the decode step, and the prefill step with its own
grouped-GEMM roofline (one MFMA pass on the codes; flops counted as for the exact
layer) and its speedup over the exact prefill step.

The 64-token batch and the 235b-shaped layer are timed as whole steps, each with
the roofline of its own dominant kernels, under "others". For context,
hbm_step.plain_read_probe times a plain read-only device reduction (torch) of 7,
14 and 21 MiB (the decode kernels' weight bytes) the same way: one HIP graph
cycling over >= 1 GB of sources, so each read comes from HBM.

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
X_POOL = 64                    # distinct input batches per replica for T <= POOL_MAX_T
POOL_MAX_T = 64
SMALL_BUCKET = 16              # buckets of at most this many pairs take the 16-row GEMM
DTYPE = "q4k x fp32 (fp16 hi+lo MFMA, fp32 acc; fp64 router)"


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
    ap.add_argument("--no-q8", action="store_true", help="skip timing the int8-activation variant")
    ap.add_argument("--no-probe", action="store_true", help="skip the plain read probe")
    ap.add_argument("--no-steps-dist", action="store_true", help="skip the single-step warm/cold distribution")
    ap.add_argument("--extra-workloads", default="30b-batch,235b-shape",
                    help="comma-separated workloads whose step time and kernel rooflines go under \"others\" "
                         "('' for none)")
    ap.add_argument("--extra-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--stages", action="store_true", help="also time every stage (eager pass, to stderr)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


def upload_layer(inp):
    """The layer of one replica's host inputs, and its input batch on the device."""
    import torch

    import quantized_moe_wave_amd as q

    wl = inp.wl
    layer = q.MoeFfn.from_host(wl.hidden, wl.experts, wl.top_k, wl.inter, inp.gate, inp.up, inp.down, inp.router,
                               inp.bias)
    return layer, torch.from_numpy(inp.x).cuda()


class Bench:
    """R replicas of one workload on the GPU (each with a pool of P input batches), outputs preallocated."""

    def __init__(self, wl, replicas: int, seed: int = 1, block: bool = False, q8: bool = False):
        import torch

        import synth

        self.wl = wl
        self.block = block
        self.q8 = q8
        self.P = X_POOL if wl.tokens <= POOL_MAX_T else 1
        self.layers, self.xs, self.outs, self.ws, self.idxs = [], [], [], [], []
        self.host0 = None
        for r in range(replicas):
            log(f"{wl.name}: generating replica {r + 1}/{replicas}")
            inp = synth.make_inputs(wl, seed=seed, replica=r)
            layer, x = upload_layer(inp)
            layer.reserve(wl.tokens)
            if block:
                layer.set_norm(torch.from_numpy(synth.gen_norm(seed, r, wl.hidden)), synth.NORM_EPS)
            # pool entry 0 is the replica's own x; the others are further seeded draws of the same distribution
            pool = [x] + [torch.from_numpy(synth.gen_x(seed + 1000 + p, r, wl.tokens, wl.hidden)).cuda()
                          for p in range(1, self.P)]
            if r == 0:
                self.host0 = inp
            self.layers.append(layer)
            self.xs.append(pool)
            self.outs.append(torch.empty_like(x))
            self.ws.append(torch.empty((wl.tokens, wl.top_k), dtype=torch.float32, device=x.device))
            self.idxs.append(torch.empty((wl.tokens, wl.top_k), dtype=torch.int32, device=x.device))
        torch.cuda.synchronize()

    @property
    def R(self):
        return len(self.layers)

    def slot(self, i: int):
        """(replica, pool entry) of step i."""
        return i % self.R, (i // self.R) % self.P

    def step(self, i: int) -> None:
        r, p = self.slot(i)
        x = self.xs[r][p]
        if self.block:
            self.layers[r].forward_block(x, self.outs[r], self.ws[r], self.idxs[r])
        elif self.q8:
            self.layers[r].forward_q8(x, self.outs[r], self.ws[r], self.idxs[r])
        else:
            self.layers[r].forward(x, self.outs[r], self.ws[r], self.idxs[r])

    def routing(self):
        """Per (replica, pool entry): its expert counts (from the layer's own routing)."""
        import numpy as np
        import torch

        self.counts = {}
        for r in range(self.R):
            for p in range(self.P):
                self.step(r + self.R * p)
                torch.cuda.synchronize()
                idx = self.idxs[r].cpu().numpy()
                self.counts[(r, p)] = np.bincount(idx.ravel(), minlength=self.wl.experts)
        return self.counts

    def step_stats(self, i: int) -> dict:
        """Routing figures of step i: distinct experts U, largest bucket, pairs in 64-row GEMM buckets, experts
        in 16-row buckets."""
        c = self.counts[self.slot(i)]
        return {"U": int((c > 0).sum()), "max": int(c.max()), "rows_big": int(c[c > SMALL_BUCKET].sum()),
                "small": int(((c > 0) & (c <= SMALL_BUCKET)).sum())}

    def touched(self, steps: int) -> dict:
        """Union of experts touched per replica over steps 0..steps-1, and their weight bytes."""
        import numpy as np

        seen = [np.zeros(self.wl.experts, bool) for _ in range(self.R)]
        for i in range(steps):
            r, p = self.slot(i)
            seen[r] |= self.counts[(r, p)] > 0
        per = [int(s.sum()) for s in seen]
        return {"experts_per_replica": per, "bytes": int(sum(per) * self.wl.expert_bytes)}

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
        """{stage: (total ms, launches)} from kernel-stamped events over eager steps 0..steps-1."""
        import torch

        import quantized_moe_wave_amd as q

        for layer in self.layers:
            q.moe_ffn_profile(layer.handle, stages)
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        res = {s: [0.0, 0] for s in stages}
        for layer in self.layers:
            got = q.moe_ffn_profile_read(layer.handle)
            q.moe_ffn_profile(layer.handle, [])
            for s in stages:
                res[s][0] += got[s][0]
                res[s][1] += got[s][1]
        return res

    def close(self):
        for layer in self.layers:
            layer.close()
        self.layers = []


def profile_record(kernel: str, workload: str, which: str):
    """Per-dispatch counter figures of `kernel` on `workload` committed under profiles/ (which = "traffic": HBM bytes
    from rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by the plain-copy calibration; "sq": MFMA-busy and VALU figures
    from SQ counters), or None if not measured on that workload or if the kernel's sources changed since (hash of
    the listed files). Records are keyed "<kernel> @ <workload>": the figures depend on the routing."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", "hbm_traffic.md" if which == "traffic" else "sq_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    k = data["kernels"].get(f"{kernel} @ {workload}")
    if k is None:
        return None
    h = hashlib.sha256()
    for f in k["files"]:
        h.update(open(os.path.join(ROOT, "quantized_moe_wave_amd", "csrc", f), "rb").read())
    if h.hexdigest()[:16] != k["source_hash"]:
        return None
    if which == "traffic":
        return int(round((k["fetch_kib"] * data["fetch_factor"] + k["write_kib"] * data["write_factor"]) * 1024))
    return {key: k[key] for key in ("mfma_busy", "valu_per_mfma") if key in k}


def replicas_for(wl) -> int:
    layer_bytes = wl.experts * wl.expert_bytes + wl.experts * wl.hidden * 4
    return max(1, math.ceil(REPLICA_BYTES / layer_bytes))


def gate_up_bytes_per_expert(wl) -> int:
    return 2 * wl.hidden * wl.inter * 144 // 256


# The kernels a roofline can be reported for: (stage names summed per step, bound, profile key)
KERNELS = {
    "decode": (["gate_up"], "hbm", "gateup_pair_kernel"),
    "small": (["gate_up"], "hbm", "expert_gemm_kernel<gate_up, 16-row tiles>"),
    "big": (["gate_up_big", "gate_up_tail"], "mfma", "expert_gemm_kernel<gate_up, 64-row tiles>"),
}


def kernel_roofline(b: Bench, steps: int, kind: str) -> dict | None:
    """Roofline of one gate/up kernel over `steps` eager steps: algorithmic work of every launch / its
    kernel-stamped time. decode: the per-pair decode kernel, bytes = U * routed gate+up bytes per expert; small: the
    16-row grouped GEMM, bytes = (experts with 1..16 pairs) * gate+up bytes per expert; big: the 64-row grouped GEMM
    (its 8-wave launch + the launch of the last-round halves), flops = 2 * rows * 2I * H."""
    import quantized_moe_wave_amd as q

    stages, bound, pkey = KERNELS[kind]
    if b.q8:
        pkey += " on Q8_K codes"  # a kernel of its own: no stored counters apply
    stages = [s for s in stages if s in q.moe_ffn_stage_names()]
    got = b.stage_times(steps, stages)
    total_ms = sum(got[s][0] for s in stages)
    launches = got[stages[0]][1]
    if launches == 0 or total_ms <= 0:
        return None
    wl = b.wl
    st = [b.step_stats(i) for i in range(steps)]
    if bound == "hbm":
        per = "U" if kind == "decode" else "small"
        work = sum(s[per] for s in st) * gate_up_bytes_per_expert(wl)
        achieved = work / (total_ms * 1e-3) / 1e9
        rec = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profile_record(pkey, wl.name, "traffic"),
               "algorithmic_bytes_per_launch": int(round(work / launches))}
    else:
        work = sum(2.0 * s["rows_big"] * 2 * wl.inter * wl.hidden for s in st)
        achieved = work / (total_ms * 1e-3) / 1e12
        rec = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": profile_record(pkey, wl.name, "traffic"),
               "algorithmic_flops_per_launch": round(work / launches)}
        sq = profile_record(pkey, wl.name, "sq")
        if sq:
            rec.update(sq)
    rec["kernel"] = f"{pkey} ({' + '.join(stages)})"
    rec["avg_us"] = round(total_ms / launches * 1e3, 3)
    log(f"{wl.name}: {rec['kernel']} avg {rec['avg_us']:.2f} us/launch -> {rec['achieved']} {rec['unit']} "
        f"({rec['frac']:.3f} of peak)")
    return rec


def kinds_for(b: Bench):
    """Roofline kernels of a workload, dominant first."""
    if b.wl.tokens <= 4:
        return ["decode"]
    st = [b.step_stats(i) for i in range(b.R * b.P)]
    has_big = any(s["rows_big"] for s in st)
    has_small = any(s["small"] for s in st)
    return (["big"] if has_big else []) + (["small"] if has_small else [])


def log_stages(b: Bench, steps: int) -> None:
    import quantized_moe_wave_amd as q

    for s, (tm, n) in b.stage_times(steps, q.moe_ffn_stage_names()).items():
        if n:
            log(f"{b.wl.name}: stage {s:12s} {tm / n * 1e3:9.2f} us avg over {n} launches")


def measure(wl, steps: int, warmup: int, eager: bool, want_stages: bool, dist: bool = True,
            q8: bool = False) -> dict:
    """Step time, the roofline of the workload's kernels, the experts touched, and the single-step distribution
    (q8: of moe_ffn_forward_q8)."""
    import torch

    b = Bench(wl, replicas_for(wl), q8=q8)
    try:
        b.routing()
        ms = b.timed(steps, warmup, eager)
        st = [b.step_stats(i) for i in range(steps)]
        U = sum(s["U"] for s in st) / steps
        touched = b.touched(steps)
        log(f"{wl.name}{' q8' if q8 else ''}: {ms * 1e3:.2f} us/step over {steps} steps ({'eager' if eager else 'graph'}); "
            f"mean U {U:.1f}; experts touched over the loop {touched}")
        roofs = [r for r in (kernel_roofline(b, steps, k) for k in kinds_for(b)) if r]
        if want_stages:
            log_stages(b, steps)
        res = {"ms": ms, "U": U, "max_tokens_per_expert": max(s["max"] for s in st),
               "gemm_rows": sum(s["rows_big"] for s in st) / steps, "touched": touched, "roofs": roofs}
        if dist:
            res["dist"] = b.per_step(max(20, min(steps, 200)))
        res["host0"] = b.host0
        return res
    finally:
        b.close()
        del b
        torch.cuda.empty_cache()


def step_line(wl, m: dict) -> dict:
    """Throughput of a measured workload: tokens/s, routed-expert bytes and algorithmic flops against the peaks."""
    T, k, H, I, E = wl.tokens, wl.top_k, wl.hidden, wl.inter, wl.experts
    sec = m["ms"] * 1e-3
    step_bytes = m["U"] * wl.expert_bytes
    flops = 2.0 * T * k * 3 * H * I + 2.0 * T * E * H
    out = {"workload": wl.name, "tokens": T, "ms_per_step": round(m["ms"], 5), "tokens_per_s": round(T / sec, 1),
           "distinct_experts": m["U"], "max_tokens_per_expert": m["max_tokens_per_expert"],
           "hbm_step": {"routed_expert_bytes": int(step_bytes), "achieved_gbs": round(step_bytes / sec / 1e9, 1),
                        "frac": round(step_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                        "experts_touched": m["touched"]},
           "mfma_step": {"algorithmic_tflops": round(flops / sec / 1e12, 2),
                         "frac": round(flops / sec / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
           "rooflines": m["roofs"]}
    if "dist" in m:
        out["step_us"] = m["dist"]
        cold = m["dist"]["cold"]["median"] * 1e-6
        out["hbm_step"]["cold_frac"] = round(step_bytes / cold / 1e9 / HBM_PEAK_GBS, 4)
    return out


def measure_block(wl, steps: int, eager: bool) -> dict:
    """The layer inside its block (moe_ffn_forward_block: RMSNorm, the layer, residual add), timed like the main
    step, with the norm kernel's own time from kernel-stamped events."""
    import torch

    import quantized_moe_wave_amd as q

    b = Bench(wl, replicas_for(wl), block=True)
    try:
        ms = b.timed(steps, max(3, steps // 10), eager)
        tm, n = b.stage_times(steps, ["norm"])["norm"]
        norm_us = tm / max(n, 1) * 1e3
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
            "norm_launches_per_step": round(n / steps, 3), "stage_stats_us": round(stats_us, 2)}


def measure_q8(wl, steps: int, eager: bool) -> dict:
    """The layer with Q8_K-style int8 expert activations (moe_ffn_forward_q8), timed like the main step."""
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


def read_probe(sizes_mb=(7, 14, 21), steps: int = 200) -> dict:
    """Context for the decode roofline: a plain read-only reduction (torch.sum) over the decode kernels' byte
    counts, timed like a step (one HIP graph of `steps` reductions cycling over >= 1 GB of sources, so each read
    comes from HBM)."""
    import torch

    out = {}
    for mb in sizes_mb:
        n = mb * (1 << 20) // 4
        R = max(4, REPLICA_BYTES // (n * 4))
        src = [torch.randn(n, device="cuda") for _ in range(R)]
        dst = torch.empty((), device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                torch.sum(src[i % R], dim=0, out=dst)
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
    log(f"plain read probe: {out}")
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
    m = measure(wl, args.steps, args.warmup, args.eager, args.stages, dist=not args.no_steps_dist)
    host0 = m["host0"]
    ms = m["ms"]
    sl = step_line(wl, m)
    line = {
        "metric": METRIC,
        "value": round(wl.tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": wl.name, "hidden": wl.hidden, "experts": wl.experts, "top_k": wl.top_k,
                   "moe_intermediate": wl.inter, "tokens": wl.tokens, "replicas": replicas_for(wl),
                   "input_pool": X_POOL if wl.tokens <= POOL_MAX_T else 1,
                   "timing": "eager" if args.eager else "hip-graph"},
        "hbm_step": {"routed_expert_bytes": sl["hbm_step"]["routed_expert_bytes"],
                     "achieved": sl["hbm_step"]["achieved_gbs"], "unit": "GB/s",
                     "frac": sl["hbm_step"]["frac"], "cold_frac": sl["hbm_step"].get("cold_frac"),
                     "distinct_experts": m["U"], "experts_touched": m["touched"]},
        "roofline": m["roofs"][0] if m["roofs"] else None,
        "other_rooflines": m["roofs"][1:],
    }
    if "step_us" in sl:
        line["step_us"] = sl["step_us"]
    if not args.no_prefill:
        pw = synth.WORKLOADS[args.prefill_workload]
        pm = measure(pw, args.prefill_steps, max(3, args.prefill_steps // 10), args.eager, args.stages,
                     dist=not args.no_steps_dist)
        pl = step_line(pw, pm)
        line["prefill"] = dict(pl, steps=args.prefill_steps, tflops=pl["mfma_step"]["algorithmic_tflops"],
                               frac_mfma_peak=pl["mfma_step"]["frac"], gemm_rows=pm["gemm_rows"],
                               roofline=pm["roofs"][0] if pm["roofs"] else None)
    if not args.no_block:
        line["block"] = [measure_block(wl, args.steps, args.eager)]
        if not args.no_prefill:
            line["block"].append(measure_block(synth.WORKLOADS[args.prefill_workload], args.prefill_steps, args.eager))
    if not args.no_q8:
        q8s = []
        if wl.tokens <= 4:
            q8s.append(measure_q8(wl, args.steps, args.eager))
        if not args.no_prefill:
            qm = measure(pw, args.prefill_steps, max(3, args.prefill_steps // 10), args.eager, args.stages,
                         dist=False, q8=True)
            ql = step_line(pw, qm)
            q8s.append(dict(ql, steps=args.prefill_steps, tflops=ql["mfma_step"]["algorithmic_tflops"],
                            frac_mfma_peak=ql["mfma_step"]["frac"], speedup_vs_exact=round(pm["ms"] / qm["ms"], 3),
                            roofline=qm["roofs"][0] if qm["roofs"] else None))
        line["q8_activations"] = q8s
    if not args.no_probe:
        line["hbm_step"]["plain_read_probe"] = read_probe()
    extras = [w for w in args.extra_workloads.split(",") if w]
    if extras:
        line["others"] = []
        for name in extras:
            ow = synth.WORKLOADS[name]
            om = measure(ow, args.extra_steps, max(3, args.extra_steps // 10), args.eager, args.stages, dist=False)
            line["others"].append(dict(step_line(ow, om), steps=args.extra_steps))
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {wl.name} for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(host0, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
