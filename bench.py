#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
    python bench.py --prefill-only | --decode-t4-only | --convert-only
    python bench.py --ceilings | --calibrate-copy | --summarize-rocprof DIR
                                      (measurement and profiling helpers)

Default workload: the GLM-5.2-shaped decode stack -- 12 resident layers of
H=6144, 256 routed experts of I=2048 + 1 shared expert (int4, gs64 fp16
scales, about 58 GiB in HBM), top-8 sigmoid routing with renormalised
weights and a Zipf-skewed router, one token.  A step is one pass of the hot
path through all 12 layers: route (top-k + grouping) and the decode forward
(gate/up GEMV + SwiGLU, down GEMV, combine) per layer, captured once in HIP
graphs and replayed; router logits rotate across 8 pre-generated sets so
successive steps stream different experts (the 12-layer working set of
2.2 GB per step dwarfs the 256 MB Infinity Cache).

value = MoE-layer tokens/s = tokens x layers / step time.  Also reported:
int4 weight GB/s of the whole step (algorithmic bytes: every distinct expert
of each layer's batch union, plus the shared expert, read once), the
roofline of the dominant kernel (decode gate/up GEMV: algorithmic bytes per
launch over its average duration from HIP events; also against a plain read
of 120 MB timed in the same run), the CPU oracle on a bounded sample, and secondary workloads (decode at 4 tokens, the 2048-token
GLM prefill on int8 matrix cores, the router GEMV, the weight quantisers,
OLMoE-like and 35B-A3B-class layers, int8 and MXFP4 expert containers).

Prints ONE JSON line.  Inputs are synthetic (seeded generator module
`synth`); all inputs are resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 matrix peak (POP/s -> TOPS)
FP8_PEAK_TOPS = 5000.0     # MI355X dense fp8 matrix peak; E2M1 x E4M3 runs at this rate
# fp32 vector peak; a bf16 dot2 (two products and two adds per lane) issues
# at the same rate as a packed fp32 FMA, so it is the dot2 router's ALU peak
FP32_VECTOR_PEAK_TFLOPS = 157.3
METRIC = "MoE-layer tokens/s + int4 weight GB/s (decode) / int8 TOPS (prefill)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class DecodeStack:
    """L resident layers of one shape; captures one graph per logit rotation."""

    def __init__(self, spec, layers, T, zipf, rotations=8, seed=0, layer_weights=None):
        import torch

        import int4_routed_expert_router_amd as coli
        import synth

        self.spec, self.L, self.T = spec, layers, T
        self.layers = layer_weights or [
            coli.Layer.from_spec(spec, *synth.make_weights(spec, seed=seed, layer=l, device="cuda"))
            for l in range(layers)]
        self.x = [synth.make_x(spec, T, seed=seed, layer=l).cuda() for l in range(layers)]
        self.logits = [[synth.make_logits(spec, T, seed=seed, layer=l, zipf_alpha=zipf,
                                          step=r).cuda() for l in range(layers)]
                       for r in range(rotations)]
        self.route = coli.Route(self.layers[0], T)
        self.ws = coli.workspace(self.layers[0], T, coli.COLI_ENTRY_DECODE)
        self.y = [torch.empty(T, spec.hidden, dtype=torch.bfloat16, device="cuda")
                  for _ in range(layers)]
        self.graphs = []
        self.coli = coli

    def step_eager(self, rot):
        c = self.coli
        for l in range(self.L):
            c.coli_moe_route(self.layers[l], self.logits[rot][l], None, self.T, self.route)
            c.coli_moe_forward_decode(self.layers[l], self.route, self.x[l], self.T, self.y[l],
                                      c.COLI_OUT_BF16, self.ws)

    def capture(self):
        import torch

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step_eager(0)  # warm the launch path before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for r in range(len(self.logits)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step_eager(r)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self, i):
        self.graphs[i % len(self.graphs)].replay()


def union_bytes(spec, logits_list, k):
    """Algorithmic weight bytes of one step: per layer, every distinct routed
    expert of the batch plus the shared expert, each read once."""
    import torch

    total = 0
    for lg in logits_list:
        idx = torch.topk(lg.float(), k, dim=1).indices  # selection only: counts experts
        n = int(torch.unique(idx).numel()) + spec.n_shared
        total += n * spec.expert_total_bytes
    return total


def time_graph(stack, warmup, steps):
    import torch

    for i in range(warmup):
        stack.replay(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        stack.replay(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def traced_kernels(fn, reps):
    """Run fn() reps times eagerly with the library's kernel timer on: each
    kernel's dispatch stamps its own start/stop events, so the spans are the
    kernels' execution times (they agree with rocprofv3's kernel trace)."""
    import torch

    import int4_routed_expert_router_amd as coli

    timer = coli.KernelTimer(capacity=max(4096, 64 * reps))
    torch.cuda.synchronize()
    with timer:
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    res = timer.results()
    timer.close()
    by = {}
    for name, ms in res:
        by.setdefault(name, []).append(ms)
    return {k: {"n": len(v), "avg_us": 1e3 * statistics.mean(v)} for k, v in by.items()}


# ------------------------------------------------------ measured HBM traffic

TRAFFIC_PROFILE = os.path.join(_ROOT, "profiles", "decode_gateup_glm52_stack_traffic.md")
KERNEL_SOURCES = ("int4_routed_expert_router_amd/csrc/decode_stream.hip",
                  "int4_routed_expert_router_amd/csrc/codec.h",
                  "int4_routed_expert_router_amd/csrc/device_common.h",
                  "int4_routed_expert_router_amd/csrc/internal.h")


def kernel_digest():
    """sha256 over the sources of the single-token decode kernels."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(_ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary, or None if it is missing or the kernel changed since."""
    import re

    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    dig = re.search(r"kernel source digest:\s*`?([0-9a-f]{16})", text)
    val = re.search(r"traffic bytes per launch:\s*`?([0-9]+)", text)
    if not dig or not val or dig.group(1) != kernel_digest():
        return None
    return int(val.group(1))


def calibrate_copy(mib=256, reps=5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def summarize_rocprof(path):
    """Per-kernel summary (markdown) of a rocprofv3 csv output directory:
    kernel-trace stats, or the mean of each counter per dispatch."""
    import collections
    import csv
    import glob
    import re

    def short(n):
        n = n.replace("coli::(anonymous namespace)::", "").replace("void ", "")
        return re.sub(r"\(.*", "", n)

    stats = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    pmc = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if stats:
        print("| kernel | calls | average (us) | min (us) | max (us) | share |")
        print("|---|---|---|---|---|---|")
        for r in csv.DictReader(open(stats[0])):
            print("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
                short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    for f in pmc:
        acc = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(f)):
            acc[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
        print("| kernel | dispatches | counter | mean per dispatch |")
        print("|---|---|---|---|")
        for k, cs in acc.items():
            for c, v in cs.items():
                print("| `%s` | %d | %s | %.1f |" % (k, len(v), c, statistics.mean(v)))


def read_ceiling(sizes_mb=(60, 120), buffers=8, reps=40):
    """The plain streaming-read rate of this chip, for the roofline fractions:
    coli_moe_read_probe (the decode GEMVs' access pattern without their
    arithmetic) over `buffers` rotating buffers per size, so that successive
    reads miss the 256 MB Infinity Cache, timed per dispatch."""
    import torch

    import int4_routed_expert_router_amd as coli

    out = {}
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for mb in sizes_mb:
        n = mb * 1000 * 1000
        bufs = [torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
                for _ in range(buffers)]
        state = {"i": 0}

        def one():
            coli.coli_moe_read_probe(bufs[state["i"] % buffers], n, sink)
            state["i"] += 1

        for _ in range(buffers):
            one()
        t = traced_kernels(one, reps)["read_probe"]
        out["%d MB" % mb] = {"bytes": n, "launches": t["n"], "avg_us": round(t["avg_us"], 2),
                             "GB_per_s": round(n / (t["avg_us"] * 1e3), 1)}
        del bufs
        torch.cuda.empty_cache()
    return {"measurement": "plain streaming read, coli_moe_read_probe", "buffers": buffers,
            "results": out, "spec_peak_GB_per_s": 8000.0}


# dense peaks of the MI355X spec sheet, per instruction's data type
MFMA_SPEC_PEAK_T = {"i8_16x16x32": 5000.0, "i8_16x16x64": 5000.0, "bf16_16x16x32": 2500.0}


def mfma_ceiling(workgroups=2048, iters=2048, reps=10):
    """The issue rate of the matrix-core instructions the kernels use, with no
    memory traffic (coli_moe_mfma_probe): T(FL)OP/s per instruction, next to
    the dense spec peak of its data type."""
    import torch

    import int4_routed_expert_router_amd as coli

    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = {}
    for name, kind in (("i8_16x16x32", coli.COLI_MFMA_I8_K32),
                       ("i8_16x16x64", coli.COLI_MFMA_I8_K64),
                       ("bf16_16x16x32", coli.COLI_MFMA_BF16_K32)):
        ops = coli.coli_moe_mfma_probe(kind, iters, workgroups, sink)
        t = traced_kernels(lambda: coli.coli_moe_mfma_probe(kind, iters, workgroups, sink),
                           reps)["mfma_probe"]
        rate = ops / (t["avg_us"] * 1e-6) / 1e12
        out[name] = {"ops_per_launch": ops, "avg_us": round(t["avg_us"], 2),
                     "T_per_s": round(rate, 1), "spec_peak_T_per_s": MFMA_SPEC_PEAK_T[name],
                     "frac_of_spec": round(rate / MFMA_SPEC_PEAK_T[name], 4)}
    return {"measurement": "register-only matrix-core loop, coli_moe_mfma_probe",
            "workgroups": workgroups, "iters": iters, "results": out}


def cpu_host():
    """Host CPU model and thread count, recorded with the CPU baseline."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline_decode(spec, layers_obj, x_list, logits_list, budget_s=12.0):
    """The CPU oracle on a bounded sample of the decode stack (T = 1)."""
    import numpy as np

    import oracle
    import synth

    done, t_total = 0, 0.0
    T = x_list[0].shape[0]
    for l in range(len(layers_obj)):
        lg = logits_list[l].cpu().numpy()
        # only the experts the token uses are copied to the host (not timed)
        r0 = oracle.route(lg, spec.top_k, spec.flags, spec.routed_scale)
        used = sorted(set(int(e) for e in r0["topk_idx"].ravel()))
        experts = used + ([spec.n_experts] if spec.n_shared else [])
        q4h, sch = synth.expert_slice(spec, layers_obj[l].q4, layers_obj[l].scales, experts)
        remap = np.zeros(spec.n_experts, np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        xb = synth.bf16_bits(x_list[l])
        t0 = time.perf_counter()
        r = oracle.route(lg, spec.top_k, spec.flags, spec.routed_scale)
        oracle.forward_decode(spec.hidden, spec.inter, len(used), spec.n_shared, spec.top_k,
                              q4h, sch, remap[r["topk_idx"]], r["topk_w"], xb)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    # with fewer tokens than threads the oracle splits each token's output
    # rows across its OpenMP threads, so every thread works
    cores = oracle.threads()
    return {"value": T * done / t_total, "unit": "MoE-layer tokens/s", "cores": cores,
            "kind": "oracle", "host": cpu_host(),
            "sample": "%d of the 12 layers, %d token(s) each, route + decode-mode layer in fp64 "
                      "(%.1f s)" % (done, T, t_total)}


def cpu_baseline_prefill(spec, layer, lg, x, T, budget_s=12.0, chunk=32):
    """The CPU oracle on a bounded token sample of a prefill workload: the
    integer-path layer (Q8_0, exact block dots, fp64 sums) for the first
    tokens of the batch, in chunks of `chunk` tokens until about `budget_s`
    seconds have run."""
    import numpy as np

    import oracle
    import synth

    lgh = lg.cpu().numpy()
    q4h, sch = synth.expert_slice(spec, layer.q4, layer.scales, list(range(spec.n_total)))
    xb = synth.bf16_bits(x)
    done, t_total = 0, 0.0
    while done < T and t_total < budget_s:
        n = min(chunk, T - done)
        t0 = time.perf_counter()
        r = oracle.route(lgh[done:done + n], spec.top_k, spec.flags, spec.routed_scale)
        oracle.forward_prefill(spec.hidden, spec.inter, spec.n_experts, spec.n_shared,
                               spec.top_k, q4h, sch, r["topk_idx"], r["topk_w"],
                               xb[done:done + n], weights=spec.weights)
        t_total += time.perf_counter() - t0
        done += n
    ops = 2.0 * 3 * spec.hidden * spec.inter * done * (spec.top_k + spec.n_shared)
    return {"value": done / t_total, "unit": "prefill tokens/s", "cores": oracle.threads(),
            "kind": "oracle", "int8_ops_per_s": round(ops / t_total, 1),
            "sample": "the first %d of %d tokens, route + integer-path layer in fp64 (%.1f s)"
                      % (done, T, t_total)}


def secondary_decode(name, spec, T, zipf, layers, steps, warmup, layer_weights=None):
    stack = DecodeStack(spec, layers, T, zipf, layer_weights=layer_weights)
    stack.capture()
    ms, _ = time_graph(stack, warmup, steps)
    nbytes = statistics.mean(union_bytes(spec, stack.logits[r], spec.top_k)
                             for r in range(len(stack.logits)))
    gbps = nbytes / (ms * 1e-3) / 1e9
    # per-kernel times per layer, from dispatch-stamped events over eager steps
    kern = traced_kernels(lambda: stack.step_eager(1), reps=4)
    return {"workload": name, "path": "decode", "weights": spec.weights,
            "tokens": T, "layers": layers,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(T * layers / (ms * 1e-3), 1),
            "weight_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()}}


def secondary_prefill(name, spec, T, zipf, steps, warmup, layer=None, copies=1,
                      k32_ceiling=None, cpu=False):
    import torch

    import int4_routed_expert_router_amd as coli
    import synth

    Ls = [layer] if layer is not None else [
        coli.Layer.from_spec(spec, *synth.make_weights(spec, seed=0, layer=c, device="cuda"))
        for c in range(copies)]
    lg = synth.make_logits(spec, T, seed=0, zipf_alpha=zipf).cuda()
    x = synth.make_x(spec, T, seed=0).cuda()
    r = coli.Route(Ls[0], T)
    ws = coli.workspace(Ls[0], T, coli.COLI_ENTRY_PREFILL)
    y = torch.empty(T, spec.hidden, dtype=torch.bfloat16, device="cuda")

    def step(i):
        L = Ls[i % len(Ls)]
        coli.coli_moe_route(L, lg, None, T, r)
        coli.coli_moe_forward_prefill(L, r, x, T, y, coli.COLI_OUT_BF16, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kern = traced_kernels(lambda: step(0), reps=3)
    nbytes = union_bytes(spec, [lg], spec.top_k)
    ops = 2.0 * 3 * spec.hidden * spec.inter * T * (spec.top_k + spec.n_shared)
    gemm_us = sum(kern.get(k, {"avg_us": 0})["avg_us"] for k in ("gemm_gateup", "gemm_down"))
    # the matrix-core format the GEMMs run in: int8 (Q8_0 activations) or the
    # scaled MX instruction (E2M1 weights x E4M3 activations, the fp8 rate)
    fmt, peak = ("mx", FP8_PEAK_TOPS) if spec.mx_act else ("int8", INT8_PEAK_TOPS)
    out = {"workload": name, "path": "prefill",
           "weights": spec.weights, "tokens": T, "ms_per_step": round(ms, 4),
           "activations": "mxfp8 (MX matrix cores)" if spec.mx_act else "q8_0 (int8 matrix cores)",
           "tokens_per_s": round(T / (ms * 1e-3), 1),
           fmt + "_TOPS": round(ops / (ms * 1e-3) / 1e12, 2),
           fmt + "_frac": round(ops / (ms * 1e-3) / 1e12 / peak, 4),
           "gemm_" + fmt + "_TOPS": round(ops / (gemm_us * 1e-6) / 1e12, 2) if gemm_us else None,
           "weight_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
           "kernels_us_from": "3 eager steps after the timed ones, each kernel's dispatch events"}
    if k32_ceiling:  # the measured rate of the instruction the GEMM issues
        out["measured_k32_TOPS"] = k32_ceiling
        out["frac_of_measured_k32"] = round(ops / (ms * 1e-3) / 1e12 / k32_ceiling, 4)
    if cpu:
        out["cpu_baseline"] = cpu_baseline_prefill(spec, Ls[0], lg, x, T)
    return out


def prefill_dense(steps, warmup):
    """The prefill GEMMs above the ridge: a GLM-shaped layer (H 6144, I 2048)
    with one routed expert (top-1) and the shared expert, so that both see
    all 2048 tokens: 32 full 64-token tiles per expert, the shape of the
    shared expert's GEMM in every prefill batch."""
    import synth

    spec = synth.LayerSpec(6144, 2048, 1, 1, 1, sigmoid=True, renorm=True)
    out = secondary_prefill("glm_shape_dense_2experts_T2048", spec, 2048, 0.0, steps, warmup)
    out["note"] = "routed expert 0 and the shared expert each take all 2048 tokens"
    return out


def prefill_dense_mx(steps, warmup):
    """The same two dense GEMMs with MXFP4 experts on the MX path (MXFP8
    activations, block scales applied by the scaled matrix-core instruction)."""
    import synth

    spec = synth.LayerSpec(6144, 2048, 1, 1, 1, sigmoid=True, renorm=True, mxfp4=True,
                           mx_act=True)
    out = secondary_prefill("glm_shape_dense_2experts_mxfp4_mx_T2048", spec, 2048, 0.0, steps,
                            warmup)
    out["note"] = "routed expert 0 and the shared expert each take all 2048 tokens"
    return out


def secondary_router(name, spec, T, steps, warmup):
    """Router logits + routing from the layer input (coli_moe_route_hidden)."""
    import torch

    import int4_routed_expert_router_amd as coli
    import synth

    small = synth.LayerSpec(spec.hidden, 64, spec.n_experts, spec.n_shared, spec.top_k,
                            spec.sigmoid, spec.renorm, spec.routed_scale)
    q4, sc = synth.make_weights(small, seed=0, device="cuda", experts=1)
    L = coli.Layer(spec.hidden, 64, spec.n_experts, spec.n_shared, spec.top_k, spec.flags, q4,
                   sc, spec.routed_scale)
    copies = 8  # rotate router weights so repeated calls do not hit in cache
    ws = [synth.make_router_weights(spec, seed=0, layer=c, device="cuda") for c in range(copies)]
    x = synth.make_x(spec, T, seed=0).cuda()
    r = coli.Route(L, T)
    logits = torch.empty(T, spec.n_experts, dtype=torch.float32, device="cuda")

    def step(i):
        coli.coli_moe_route_hidden(L, ws[i % copies], x, None, T, logits, r)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kern = traced_kernels(lambda: step(1), reps=max(4, steps // 4))
    us = kern["router_logits"]["avg_us"]
    wbytes = spec.n_experts * spec.hidden * 2
    flops = 2.0 * T * spec.n_experts * spec.hidden
    return {"workload": name, "path": "router", "tokens": T, "ms_per_call": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1),
            "router_logits_us": round(us, 3),
            "router_weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
            "router_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
            "alu_frac": round(flops / (us * 1e-6) / 1e12 / FP32_VECTOR_PEAK_TFLOPS, 4),
            "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()}}


def secondary_convert(name, spec, experts, src, steps, warmup, fmt="int4"):
    """Float weights -> an expert container (int4 gs64, int8 gs64 or MXFP4:
    coli_moe_quantize_int4_gs64 / _int8_gs64 / coli_moe_quantize_mxfp4) for
    `experts` experts of the spec's shape stored back to back, in one call."""
    import torch

    import int4_routed_expert_router_amd as coli
    import synth

    dtype, code = {"bf16": (torch.bfloat16, coli.COLI_SRC_BF16),
                   "f32": (torch.float32, coli.COLI_SRC_F32)}[src]
    n = experts * 3 * spec.inter * spec.hidden
    w = synth.make_float_weights(n, seed=0, device="cuda", dtype=dtype)
    # codes: n/2 bytes (n for int8); scales: n/32 bytes in every format (an
    # fp16 per 64 weights, or an E8M0 byte per 32)
    q4 = torch.empty(n if fmt == "int8" else n // 2, dtype=torch.uint8, device="cuda")
    sc = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    rows = n // spec.hidden
    fn = {"int4": coli.coli_moe_quantize_int4_gs64, "int8": coli.coli_moe_quantize_int8_gs64,
          "mxfp4": coli.coli_moe_quantize_mxfp4}[fmt]

    def step(i):
        fn(w, code, rows, spec.hidden, q4, sc)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kern = traced_kernels(lambda: step(0), reps=max(4, steps // 2))
    us = kern["quantize_" + fmt]["avg_us"]
    nbytes = n * w.element_size() + q4.numel() + sc.numel()  # read once, write once
    del w, q4, sc
    return {"workload": name, "path": "convert", "weights": fmt, "experts": experts,
            "values": n, "src": src, "ms_per_call": round(ms, 4),
            "weights_per_s": round(n / (ms * 1e-3), 1),
            "quantize_us": round(us, 2),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="main workload only")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the 2048-token GLM prefill workload (for profiling it)")
    ap.add_argument("--prefill-tokens", type=int, default=2048,
                    help="tokens of the --prefill-only / --prefill-mx-only run (default 2048)")
    ap.add_argument("--prefill-mx-only", action="store_true",
                    help="the 2048-token GLM-shaped prefill with MXFP4 experts on the MX path")
    ap.add_argument("--prefill-dense-only", action="store_true",
                    help="the GLM-shaped GEMMs with every one of 2048 tokens on each expert")
    ap.add_argument("--decode-t4-only", action="store_true",
                    help="only the GLM-shaped decode stack with 4 tokens (verify batch)")
    ap.add_argument("--convert-only", action="store_true",
                    help="only the float -> int4 quantiser on 32 GLM-shaped experts")
    ap.add_argument("--ceilings", action="store_true",
                    help="time a plain streaming read (60 and 120 MB) and the matrix-core "
                         "issue rate, print them and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 csv output directory")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this routed-expert layer is built and timed on a "
              "single MI355X; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.ceilings:
        print(json.dumps({"read": read_ceiling(), "mfma": mfma_ceiling()}), flush=True)
        return
    if args.prefill_only:
        pw = synth.WORKLOADS["glm_prefill"]
        T = args.prefill_tokens
        print(json.dumps(secondary_prefill("glm_prefill_T%d" % T, pw.spec, T, pw.zipf_alpha,
                                           args.steps, args.warmup, copies=1)), flush=True)
        return
    if args.prefill_mx_only:
        pw = synth.WORKLOADS["glm_prefill"]
        spec = dataclasses.replace(pw.spec, mxfp4=True, mx_act=True)
        T = args.prefill_tokens
        print(json.dumps(secondary_prefill("glm_mxfp4_mx_prefill_T%d" % T, spec, T,
                                           pw.zipf_alpha, args.steps, args.warmup)), flush=True)
        return
    if args.prefill_dense_only:
        print(json.dumps(prefill_dense(args.steps, args.warmup)), flush=True)
        print(json.dumps(prefill_dense_mx(args.steps, args.warmup)), flush=True)
        return
    if args.decode_t4_only:
        w = synth.WORKLOADS["glm"]
        print(json.dumps(secondary_decode("glm_decode_stack_T4", w.spec, 4, w.zipf_alpha,
                                          w.layers, args.steps, args.warmup)), flush=True)
        return
    if args.convert_only:
        for fmt in ("int4", "int8", "mxfp4"):
            print(json.dumps(secondary_convert("glm_convert_%s_32experts_bf16" % fmt,
                                               synth.WORKLOADS["glm"].spec, 32, "bf16",
                                               args.steps, args.warmup, fmt=fmt)), flush=True)
        return
    w = synth.WORKLOADS["glm"]
    spec, T, layers = w.spec, 1, w.layers
    log("generating %d layers (%.1f GiB of int4 experts)" % (layers, synth.container_gib(spec, layers)))
    stack = DecodeStack(spec, layers, T, w.zipf_alpha)
    torch.cuda.synchronize()
    log("capturing graphs")
    stack.capture()
    log("timing %d steps" % args.steps)
    ms, wall = time_graph(stack, args.warmup, args.steps)
    nbytes = statistics.mean(union_bytes(spec, stack.logits[r], spec.top_k)
                             for r in range(len(stack.logits)))
    gbps = nbytes / (ms * 1e-3) / 1e9
    value = T * layers / (ms * 1e-3)
    log("decode stack: %.3f ms/step, %.0f layer-tokens/s, %.0f GB/s" % (ms, value, gbps))

    # dominant kernel: the gate/up GEMV (two thirds of the weight bytes),
    # timed by its own dispatch events over K more steps of the same stack
    log("timing kernels over %d eager steps" % args.steps)
    kern = traced_kernels(lambda: stack.step_eager(0), reps=args.steps)
    gu = kern["decode_gateup"]
    # T = 1: one launch reads exactly k routed experts + the shared expert
    gu_bytes = (spec.top_k + spec.n_shared) * 2 * spec.inter * spec.hidden * (0.5 + 2 / 64)
    gu_gbps = gu_bytes / (gu["avg_us"] * 1e-6) / 1e9
    traffic = measured_traffic()
    roofline = {"bound": "hbm", "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "traffic_over_algorithmic": round(traffic / gu_bytes, 4) if traffic else None,
                "kernel": "decode_gateup (gateup_stream_kernel)", "bytes_per_launch": int(gu_bytes),
                "avg_us": round(gu["avg_us"], 3), "launches_timed": gu["n"],
                "kernel_source_digest": kernel_digest(),
                "kernels_us": {k: round(v["avg_us"], 3) for k, v in kern.items()}}
    # the decode GEMV as a whole: gate/up and down bytes over their summed time
    dn = kern["decode_down"]
    dn_bytes = (spec.top_k + spec.n_shared) * spec.inter * spec.hidden * (0.5 + 2 / 64)
    gemv_gbps = (gu_bytes + dn_bytes) / ((gu["avg_us"] + dn["avg_us"]) * 1e-6) / 1e9
    roofline["decode_gemv_combined"] = {
        "kernels": "decode_gateup + decode_down", "bytes_per_layer": int(gu_bytes + dn_bytes),
        "avg_us": round(gu["avg_us"] + dn["avg_us"], 3), "achieved": round(gemv_gbps, 1),
        "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4)}
    log("kernels (us):", roofline["kernels_us"])
    log("decode GEMV (gate/up + down): %.0f GB/s, %.1f%% of 8 TB/s" % (gemv_gbps, 100 * gemv_gbps / HBM_PEAK_GBPS))
    # the same kernel against what a plain read of 120 MB reaches on this chip
    rc = read_ceiling(sizes_mb=(120,), reps=20)["results"]["120 MB"]["GB_per_s"]
    roofline["measured_read_GBps"] = rc
    roofline["frac_of_measured_read"] = round(gu_gbps / rc, 4)
    log("plain read of 120 MB: %.0f GB/s; gate/up at %.1f%% of it" % (rc, 100 * gu_gbps / rc))

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline_decode(spec, stack.layers, stack.x, stack.logits[0])

    secondary = []
    if not args.no_secondary:
        log("secondary workloads")
        secondary.append(secondary_decode("glm_decode_stack_T4", spec, 4, w.zipf_alpha, layers,
                                          max(10, args.steps // 2), 3, layer_weights=stack.layers))
        pw = synth.WORKLOADS["glm_prefill"]
        k32 = mfma_ceiling(reps=3)["results"]["i8_16x16x32"]["T_per_s"]
        secondary.append(secondary_prefill("glm_prefill_T2048", pw.spec, 2048, pw.zipf_alpha,
                                           10, 2, layer=stack.layers[0], k32_ceiling=k32,
                                           cpu=not args.no_cpu))
        # an extra, clearly labelled run of the same layer at 16,384 tokens:
        # most experts then sit above the int8 ridge (625 ops per weight byte)
        ext = secondary_prefill("glm_prefill_T16384_extra", pw.spec, 16384, pw.zipf_alpha, 5, 2,
                                layer=stack.layers[0], k32_ceiling=k32)
        ext["note"] = ("extra run: the 2048-token GLM prefill layer at 8x the tokens, "
                       "so the expert GEMMs are compute-heavy")
        secondary.append(ext)
        del stack
        torch.cuda.empty_cache()
        secondary.append(prefill_dense(10, 2))
        torch.cuda.empty_cache()
        secondary.append(prefill_dense_mx(10, 2))
        torch.cuda.empty_cache()
        secondary.append(secondary_router("glm_router_T1", w.spec, 1, 200, 10))
        secondary.append(secondary_router("glm_router_T2048", w.spec, 2048, 20, 3))
        secondary.append(secondary_convert("glm_convert_32experts_bf16", w.spec, 32, "bf16",
                                           20, 3))
        secondary.append(secondary_convert("glm_convert_8experts_f32", w.spec, 8, "f32",
                                           20, 3))
        secondary.append(secondary_convert("glm_convert_int8_32experts_bf16", w.spec, 32, "bf16",
                                           20, 3, fmt="int8"))
        secondary.append(secondary_convert("glm_convert_mxfp4_32experts_bf16", w.spec, 32,
                                           "bf16", 20, 3, fmt="mxfp4"))
        ow = synth.WORKLOADS["olmoe"]
        secondary.append(secondary_decode("olmoe_decode_T1", ow.spec, 1, 0.0, 4, 200, 10))
        secondary.append(secondary_prefill("olmoe_prefill_T512", ow.spec, 512, 0.0, 20, 3, copies=4))
        # int8-weight experts: the OLMoE-style int8 container, and a GLM-shaped
        # MTP layer (int8 experts) verifying a 4-token draft
        o8 = dataclasses.replace(ow.spec, int8=True)
        secondary.append(secondary_decode("olmoe_int8_decode_T1", o8, 1, 0.0, 4, 200, 10))
        secondary.append(secondary_prefill("olmoe_int8_prefill_T512", o8, 512, 0.0, 20, 3,
                                           copies=4))
        g8 = dataclasses.replace(w.spec, int8=True)
        secondary.append(secondary_decode("glm_mtp_int8_decode_T4", g8, 4, w.zipf_alpha, 2,
                                          50, 5))
        # MXFP4 experts (fp4 expert families): GLM-shaped decode, OLMoE-shaped prefill
        g4 = dataclasses.replace(w.spec, mxfp4=True)
        secondary.append(secondary_decode("glm_mxfp4_decode_stack_T1", g4, 1, w.zipf_alpha, 4,
                                          100, 10))
        secondary.append(secondary_prefill("olmoe_mxfp4_prefill_T512",
                                           dataclasses.replace(ow.spec, mxfp4=True), 512, 0.0,
                                           20, 3, copies=4))
        # the MX path: MXFP8 activations on the MX matrix cores (block scales in hardware)
        secondary.append(secondary_prefill("olmoe_mxfp4_mx_prefill_T512",
                                           dataclasses.replace(ow.spec, mxfp4=True, mx_act=True),
                                           512, 0.0, 20, 3, copies=4))
        pw = synth.WORKLOADS["glm_prefill"]
        import int4_routed_expert_router_amd as coli
        mxspec = dataclasses.replace(pw.spec, mxfp4=True, mx_act=True)
        mxl = coli.Layer.from_spec(mxspec, *synth.make_weights(mxspec, seed=0, layer=0,
                                                               device="cuda"))
        secondary.append(secondary_prefill("glm_mxfp4_mx_prefill_T2048", mxspec, 2048,
                                           pw.zipf_alpha, 10, 2, layer=mxl))
        ext = secondary_prefill("glm_mxfp4_mx_prefill_T16384_extra", mxspec, 16384,
                                pw.zipf_alpha, 5, 2, layer=mxl)
        ext["note"] = ("extra run: the 2048-token GLM prefill layer (MXFP4 experts, MX path) "
                       "at 8x the tokens, so the expert GEMMs are compute-heavy")
        secondary.append(ext)
        del mxl
        torch.cuda.empty_cache()
        aw = synth.WORKLOADS["a3b"]
        for t in aw.tokens:
            secondary.append(secondary_decode("a3b_decode_T%d" % t, aw.spec, t, aw.zipf_alpha, 4,
                                              200, 10))
        for s in secondary:
            log(json.dumps(s))

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "MoE-layer tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights, bf16 x bf16 products, f32 accumulation",
        "data": "synthetic (seeded; shapes of the GLM-5.2 MoE layer)",
        "config": {"workload": "glm52_decode_stack", "hidden": spec.hidden, "inter": spec.inter,
                   "routed_experts": spec.n_experts, "shared_experts": spec.n_shared,
                   "top_k": spec.top_k, "routing": "sigmoid+renorm, Zipf-skewed logits",
                   "layers": layers, "tokens": T, "weights_GiB": round(synth.container_gib(spec, layers), 2)},
        "weight_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "stack_tokens_per_s": round(T / (ms * 1e-3), 1), "wall_s": round(wall, 3),
        "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
