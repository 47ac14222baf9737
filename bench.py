#!/usr/bin/env python3
"""Benchmark of the routed int4 MoE hot path on one MI355X.

Workloads (all over the same routed MoE layer: d=2816, f=704, 128 experts,
top-8, int4 groups of 64 with fp16 scale/bias, 30 layers, seeded synthetic
weights and inputs):

  decode   (default) batch-1 decode, all 3,840 experts resident in HBM slots
           (12.85 GB), Zipf(1.1) expert popularity per layer.  One step = one
           token through the 30 layers (route -> gate/up -> down+combine per
           layer, then the unit-RMS feedback), captured once as a HIP graph.
  batched  32 concurrent decode streams per step: route, permute, grouped
           gate/up and down GEMV over variable tokens-per-expert.
  prefill  2048 tokens through the 30 layers: route, permute, grouped int4
           GEMM on MFMA (gate/up with GELU, then down), gather combine.
  cache    batch-1 decode with a bounded cache of 64 HBM slots per layer; the
           full expert pool in pinned host memory; Markov routing (each expert
           kept with probability 0.8); misses staged on a side stream while a
           shared-path bf16 GEMV (4d x d) runs on the compute stream.

Prints one JSON line.  `value` is tokens/s; the `roofline` object covers the
dominant kernel, timed with HIP events at the kernel's own begin/end on its
stream; `cpu_baseline` is the CPU oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

D, F, E, K, NL = synth.D_MODEL, synth.D_FF, synth.N_EXPERTS, synth.TOP_K, synth.N_LAYERS
# shared expert width: the pages give none; 3776 = 4d/3 rounded up to 64 makes its three bf16
# matrices as large as the d x 4d filler GEMV (63.8 MB against 63.4 MB per layer)
F_SH = 3776
METRIC = "routed-MoE tokens/s + achieved HBM GB/s (int4 decode), MFMA util (prefill)"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16
EPS = 1e-6
CSRC = os.path.join(ROOT, "int4_routed_expert_route_amd", "csrc")

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (scaled by a 1 GiB copy's readings), keyed by the workload, for the kernel
# sources and the input recipe with this fingerprint (paths from the repository
# root); reported as null once either differs.
TRAFFIC = {
    "decode": {"sources": ('int4_routed_expert_route_amd/csrc/q4_gemv.hip', 'int4_routed_expert_route_amd/csrc/q4_lane.h', 'int4_routed_expert_route_amd/csrc/common.h', 'synth/__init__.py'),
              "sha256_16": "8e9b70a6e5078a6f", "fetch_bytes": 18094707, "write_bytes": 22528},
    "decode_fused": {"sources": ('int4_routed_expert_route_amd/csrc/decode_fused.hip', 'int4_routed_expert_route_amd/csrc/q4_lane.h', 'int4_routed_expert_route_amd/csrc/common.h', 'synth/__init__.py'),
                    "sha256_16": "8f2bae3354a96ba3", "fetch_bytes": 954526903, "write_bytes": 8174496},
    "prefill": {"sources": ('int4_routed_expert_route_amd/csrc/q4_grouped_mfma.hip', 'int4_routed_expert_route_amd/csrc/common.h', 'synth/__init__.py'),
               "sha256_16": "0f438898effa6248", "fetch_bytes": 424294437, "write_bytes": 24117024},
    "batched_f16": {"sources": ('int4_routed_expert_route_amd/csrc/q4_grouped_mfma.hip', 'int4_routed_expert_route_amd/csrc/common.h', 'synth/__init__.py'),
                   "sha256_16": "0f438898effa6248", "fetch_bytes": 102122368, "write_bytes": 369744},
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def blob_bytes():
    return 3 * D * F // 2 + 3 * D * F // 64 * 4


def gateup_expert_bytes():
    return 2 * F * D // 2 + 2 * F * (D // 64) * 4


def down_expert_bytes():
    return D * F // 2 + D * (F // 64) * 4


def decode_bytes():
    """Bytes one decode token must read: per layer the router (fp32 E x d), the
    RMSNorm weight and the 8 selected expert blobs; and per gate/up / down launch."""
    per_layer = E * D * 4 + D * 4 + K * blob_bytes()
    gateup_launch = K * gateup_expert_bytes() + D * 4 + K * F * 4
    down_launch = K * down_expert_bytes() + K * F * 4 + K * 4 + 2 * D * 4
    return per_layer, gateup_launch, down_launch


def traffic_of(workload):
    t = TRAFFIC.get(workload)
    if not t:
        return None
    try:
        src = b"".join(open(os.path.join(ROOT, n), "rb").read() for n in t["sources"])
    except OSError:
        return None
    if hashlib.sha256(src).hexdigest()[:16] != t["sha256_16"]:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def build_arena(torch, api, seed):
    """Device arena of NL * E expert blobs; slot e of layer l holds expert e."""
    dm = api.dims(D, F, E, K)
    stride = api.moe_expert_blob_bytes(dm)
    t0 = time.time()
    arena = torch.empty(NL * E * stride, dtype=torch.uint8, device="cuda")
    for l in range(NL):
        blobs = synth.expert_blobs(D, F, seed, l, range(E), threads=16)
        arena[l * E * stride:(l + 1) * E * stride].copy_(torch.from_numpy(np.concatenate(blobs)))
    torch.cuda.synchronize()
    log(f"arena {arena.numel() / 1e9:.2f} GB filled in {time.time() - t0:.1f} s")
    return arena, stride


def time_launch(api, torch, call, launch, n):
    """Average duration (us) of one call's main kernel over n eager launches
    (launch(i) enqueues the i-th on the current stream), with events recorded at
    the kernel's own begin/end."""
    durs = []
    for i in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        api.moe_profile_next_launch(call, e0, e1)
        launch(i)
        e1.synchronize()
        durs.append(e0.elapsed_time(e1) * 1000.0)
    durs = np.array(durs[2:] if len(durs) > 4 else durs)
    return float(np.mean(durs)), float(np.median(durs))


def host_cpu():
    """CPU model, physical cores and the threads this process may use (its
    affinity, capped by OMP_NUM_THREADS when that is set)."""
    model, cores = "unknown", set()
    try:
        phys = core = None
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model == "unknown":
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    return model, len(cores) or None, threads


def cpu_baseline(seed, T, budget_s, what, bias_of=None):
    """The CPU oracle (plain C++ fp32, std::thread over independent rows and
    pairs) on a bounded sample of the workload: T tokens through the layers in
    order until ~budget_s of oracle time (at most all 30); expert blob
    generation is untimed.  Scaled to tokens/s of the 30-layer stack."""
    import oracle as orc
    model, phys, threads = host_cpu()
    orc.set_threads(threads)
    x = synth.tokens(T, D, seed, stream=7 if T > 1 else 0)
    spent, done = 0.0, 0
    for l in range(NL):
        blobs = dict(zip(range(E), synth.expert_blobs(D, F, seed, l, range(E), threads=16)))
        rw = synth.router_weight(D, E, seed, l)
        nw = synth.norm_weight(D, seed, l)
        bias = synth.zipf_bias(E, seed, l) if bias_of is None else bias_of(l)
        t0 = time.perf_counter()
        x, *_ = orc.moe_layer(x, nw, rw, bias, blobs.__getitem__, D, F, K)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    per_pass = spent / done * NL
    return {"value": T / per_pass, "unit": "tokens/s", "cores": int(orc.threads()), "kind": "oracle",
            "oracle": "plain C++17 fp32 (oracle/moe_oracle.cpp), sequential sums, std::thread",
            "cpu_model": model, "physical_cores": phys,
            "sample": f"{T} token(s) through layers 0-{done - 1} of one {what} step, {spent:.1f} s of oracle time"
                      + ("" if done == NL else f", scaled x{NL / done:.2f} to the 30-layer stack")}


def graph_of(torch, fn):
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        fn()  # eager warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    return graph


def timed(torch, run, steps, warm):
    log(f"warmup {warm} steps")
    run(warm)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t_wall


def base_record(value, steps, warm, ms, dtype, workload, extra_cfg):
    cfg = {"workload": workload, "layers": NL}
    cfg.update(extra_cfg)
    return {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": warm, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": cfg}


def rounded_steps(n, period):
    return max(period, (n + period - 1) // period * period)


# ----------------------------------------------------------------------------- decode

class DecodeStack:
    """Device state of the 30-layer batch-1 decode workload."""

    def __init__(self, api, torch, seed=0, cold=False, arena=None):
        self.api, self.torch = api, torch
        self.dm = api.dims(D, F, E, K)
        self.arena, self.stride = build_arena(torch, api, seed) if arena is None else arena
        dev = "cuda"
        self.slots = torch.arange(E, dtype=torch.int32, device=dev)
        self.tables = self.slots.repeat(NL, 1).contiguous()  # [NL][E], identity slots
        self.router_w = torch.from_numpy(np.stack([synth.router_weight(D, E, seed, l) for l in range(NL)])).to(dev)
        self.norm_w = torch.from_numpy(np.stack([synth.norm_weight(D, seed, l) for l in range(NL)])).to(dev)
        self.cold = cold
        if cold:
            # control arm: step s selects experts {(8s + j + 3l) mod 128}: an expert
            # comes back only every 16 steps, so the 12.85 GB working set defeats
            # the 256 MB last-level cache
            self.period = E // K
            bias = np.zeros((self.period, NL, E), dtype=np.float32)
            for s in range(self.period):
                for l in range(NL):
                    sel = [(K * s + j + 3 * l) % E for j in range(K)]
                    bias[s, l] = synth.selection_bias(np.array(sel), E)
            self.bias = torch.from_numpy(bias).to(dev)
        else:
            self.period = 1
            self.bias = torch.from_numpy(np.stack([synth.zipf_bias(E, seed, l) for l in range(NL)])[None]).to(dev)
        self.x = torch.zeros(NL + 1, D, dtype=torch.float32, device=dev)
        self.x[0].copy_(torch.from_numpy(synth.tokens(1, D, seed)[0]))
        self.h = torch.empty(1, D, dtype=torch.float32, device=dev)
        self.idx = torch.zeros(self.period, NL, K, dtype=torch.int32, device=dev)
        self.w = torch.zeros(self.period, NL, K, dtype=torch.float32, device=dev)
        self.act = torch.empty(K, F, dtype=torch.float32, device=dev)
        self.y_probe = torch.empty(1, D, dtype=torch.float32, device=dev)
        ws = lambda c: torch.zeros(max(api.moe_workspace_size(c, 1, self.dm), 256), dtype=torch.uint8, device=dev)
        self.ws_route, self.ws_gateup, self.ws_down = ws(0), ws(2), ws(3)
        self.ws_fused = torch.zeros(api.moe_workspace_size(api.MOE_CALL_DECODE_LAYERS, NL, self.dm),
                                    dtype=torch.uint8, device=dev)
        self.idx_f = torch.zeros(self.period, NL, K, dtype=torch.int32, device=dev)
        self.w_f = torch.zeros(self.period, NL, K, dtype=torch.float32, device=dev)

    def arena_of(self, l):
        return self.arena[l * E * self.stride:(l + 1) * E * self.stride]

    def fused_step(self, s, stream=None):
        """One token through the 30 layers in one launch; the unit-RMS feedback
        goes straight back into x[0]."""
        self.api.moe_decode_layers(self.x, NL, self.norm_w, EPS, self.router_w, self.bias[s], self.tables, E,
                                   self.arena, E * self.stride, self.stride, self.dm, self.idx_f[s], self.w_f[s],
                                   self.x[0], self.ws_fused, stream)

    def fused_steps(self, n_periods=1, stream=None):
        for _ in range(n_periods):
            for s in range(self.period):
                self.fused_step(s, stream)

    def route(self, s, l, stream=None):
        self.api.moe_route(self.x[l:l + 1], self.norm_w[l], EPS, self.router_w[l], self.bias[s, l], 1, self.dm,
                           self.h, self.idx[s, l:l + 1], self.w[s, l:l + 1], self.ws_route, stream)

    def gateup(self, s, l, stream=None):
        a = self.api
        a.moe_expert_q4_gateup(self.h, self.idx[s, l:l + 1], self.slots, E, self.arena_of(l), self.stride, None,
                               None, None, 0, 1, self.dm, a.MOE_PREC_FP32, self.act, self.ws_gateup, stream)

    def down(self, s, l, out, stream=None):
        a = self.api
        a.moe_expert_q4_down_combine(self.act, self.idx[s, l:l + 1], self.w[s, l:l + 1], self.slots, E,
                                     self.arena_of(l), self.stride, None, None, None, self.x[l:l + 1], 1,
                                     self.dm, a.MOE_PREC_FP32, out, self.ws_down, stream)

    def steps(self, n_periods=1, stream=None):
        for _ in range(n_periods):
            for s in range(self.period):
                for l in range(NL):
                    self.route(s, l, stream)
                    self.gateup(s, l, stream)
                    self.down(s, l, self.x[l + 1:l + 2], stream)
                self.api.moe_rms_rescale(self.x[NL:NL + 1], 1, D, EPS, self.x[0:1], stream)


def run_decode(args, api, torch):
    """The 30-layer batch-1 decode workload (Zipf routing) and its control arm
    (cold routing that defeats the last-level cache) in one invocation: after
    the warmup, timed segments alternate between the arms in both orders
    (ZC, CZ, ZC, ...), args.repeats pairs.  The Zipf segments add up to
    exactly args.steps timed steps; `value` is their overall rate, and each
    arm's per-segment median and spread are reported beside it."""
    stack = DecodeStack(api, torch, args.seed, cold=False)
    ctrl = DecodeStack(api, torch, args.seed, cold=True, arena=(stack.arena, stack.stride))
    fused = args.decode_path == "fused"
    period = stack.period
    R = max(1, args.repeats)
    seg = [args.steps // R + (1 if i < args.steps % R else 0) for i in range(R)]  # Zipf steps per segment
    cseg = rounded_steps(max(1, args.steps // R), ctrl.period)                     # control steps per segment

    def runner(st):
        body = (lambda: st.fused_steps(1)) if fused else (lambda: st.steps(1))
        if args.no_graph:
            return lambda n: [body() for _ in range(n // st.period)]
        graph = graph_of(torch, body)  # one replay = one routing period (1 step, or 16 for the control)
        return lambda n: [graph.replay() for _ in range(n // st.period)]

    run_z, run_c = runner(stack), runner(ctrl)
    log(f"warmup {args.warmup} steps per arm")
    run_z(args.warmup)
    run_c(rounded_steps(args.warmup, ctrl.period))
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def segment(run, n):
        torch.cuda.synchronize()
        e0.record()
        run(n)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0

    z_times, c_times, z_rates, c_rates = [], [], [], []
    t_wall = time.perf_counter()
    for r in range(R):
        order = ("z", "c") if r % 2 == 0 else ("c", "z")
        for arm in order:
            if arm == "z":
                if seg[r] == 0:
                    continue
                dt = segment(run_z, seg[r])
                z_times.append(dt)
                z_rates.append(seg[r] / dt)
            else:
                dt = segment(run_c, cseg)
                c_times.append(dt)
                c_rates.append(cseg / dt)
    t_wall = time.perf_counter() - t_wall
    if fused:
        api.moe_decode_check(stack.ws_fused)
        api.moe_decode_check(ctrl.ws_fused)
    steps, warm = args.steps, args.warmup
    tok_s = steps / sum(z_times)
    ms = 1000.0 / tok_s
    per_layer, gu_bytes, _ = decode_bytes()
    step_bytes = NL * per_layer
    c_tok_s = len(c_times) * cseg / sum(c_times)
    log(f"{steps} Zipf steps ({args.decode_path}) in {len(z_times)} segments: {ms * 1000:.1f} us/step, "
        f"{tok_s:.1f} tok/s (median {np.median(z_rates):.1f}, {min(z_rates):.1f}-{max(z_rates):.1f}); control "
        f"{c_tok_s:.1f} tok/s (median {np.median(c_rates):.1f}, {min(c_rates):.1f}-{max(c_rates):.1f}); "
        f"{step_bytes * tok_s / 1e9:.0f} GB/s algorithmic")

    # the step's kernels one at a time, each at its own begin/end; layer and
    # routing-period index cycle so every layer's weights are used
    sl = lambda i: ((i // NL) % period, i % NL)
    n = args.kernel_samples
    rt_us, _ = time_launch(api, torch, api.MOE_CALL_ROUTE, lambda i: stack.route(*sl(i)), n)
    gu_us, gu_med = time_launch(api, torch, api.MOE_CALL_GATEUP, lambda i: stack.gateup(*sl(i)), n)
    dn_us, _ = time_launch(api, torch, api.MOE_CALL_DOWN_COMBINE, lambda i: stack.down(*sl(i), stack.y_probe), n)
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    log(f"kernels (eager, mean us): route {rt_us:.2f}  gate/up {gu_us:.2f} (median {gu_med:.2f})  down {dn_us:.2f}")
    if fused:
        fu_us, _ = time_launch(api, torch, api.MOE_CALL_DECODE_LAYERS, lambda i: stack.fused_step(i % period), n)
        api.moe_decode_check(stack.ws_fused)
        f_achieved = step_bytes / (fu_us * 1e-6) / 1e9
        log(f"fused decode kernel (eager, mean): {fu_us:.1f} us per token, {f_achieved:.0f} GB/s algorithmic")

    out = base_record(tok_s, steps, warm, ms, "int4-fx16-fp32",
                      "batch-1 decode, 30 routed MoE layers x 128 experts (d=2816, f=704, top-8, int4 groups of "
                      "64, fp16 scale/bias), all experts resident in HBM, Zipf(1.1) routing",
                      {"tokens_per_step": 1, "graph": not args.no_graph,
                       "path": "moe_decode_layers (one launch per token)" if fused else
                               "moe_route + moe_expert_q4_gateup + moe_expert_q4_down_combine per layer"})
    out.update({
        "dtype_detail": "int4 weights (exact) x activations as 16-bit fixed point per 64-column group, exact "
                        "int32 sums inside a group, fp32 across groups; router, softmax and combine fp32",
        "protocol": {"segments": "Zipf and control alternated, orders ZC, CZ, ...", "repeats": R,
                     "zipf_tok_s": {"median": round(float(np.median(z_rates)), 1),
                                    "min": round(min(z_rates), 1), "max": round(max(z_rates), 1),
                                    "segments_steps": seg},
                     "control_tok_s": {"overall": round(c_tok_s, 1), "median": round(float(np.median(c_rates)), 1),
                                       "min": round(min(c_rates), 1), "max": round(max(c_rates), 1),
                                       "segment_steps": cseg,
                                       "routing": "step s selects experts (8s + j + 3l) mod 128: no expert "
                                                  "comes back within 16 steps (defeats the 256 MB last-level "
                                                  "cache)"}},
        "algorithmic_bytes_per_token": step_bytes,
        "algorithmic_GBps": round(step_bytes * tok_s / 1e9, 1),
        "hbm_frac_step": round(step_bytes * tok_s / 1e9 / HBM_PEAK_GBPS, 4),
        "kernel_us": {"route": round(rt_us, 3), "gateup": round(gu_us, 3), "down_combine": round(dn_us, 3)},
        "wall_s_timed": round(t_wall, 3),
    })
    if fused:
        out["kernel_us"]["decode_layers_fused"] = round(fu_us, 2)
        out["roofline"] = {
            "kernel": "k_decode_fused (30 layers of route + int4 gate/up + down + combine, one launch per token)",
            "bound": "hbm", "achieved": round(f_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(f_achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_of("decode_fused"),
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": step_bytes, "avg_launch_us": round(fu_us, 2),
        }
    else:
        out["roofline"] = {
            "kernel": "k_gateup (int4 gate/up dequant-GEMV, 8 experts, fp32 accumulate)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_of("decode"),
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 3),
        }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args.seed, 1, 20.0, "batch-1 decode (Zipf routing)")
    return out


def run_decode_timeline(args, api, torch):
    """Per-stage timeline of the fused decode kernel (measurement build
    libmoe_measure.so): every workgroup's clock at the end of each stage of
    each layer, over several eager launches after the warmup, summarised as
    markdown into args.decode_timeline."""
    import ctypes
    lib = api.lib()
    fn = lib.moe_debug_decode_timeline
    fn.argtypes = [ctypes.c_void_p]
    stack = DecodeStack(api, torch, args.seed, cold=args.control == "cold")
    for i in range(args.warmup):
        stack.fused_step(i % stack.period)
    torch.cuda.synchronize()
    G = K * F // 32  # workgroups of the launch (32 act columns each)
    tl = np.zeros((64, 256, 12), dtype=np.uint64)
    runs = []
    for i in range(args.steps):
        stack.fused_step((args.warmup + i) % stack.period)
        torch.cuda.synchronize()
        assert fn(tl.ctypes.data) == 0
        runs.append(tl[:NL, :G].astype(np.int64).copy())
    api.moe_decode_check(stack.ws_fused)
    us = 0.01  # s_memrealtime ticks at 100 MHz
    names = ["router partials, sums of squares, x arrived", "logits + top-k", "h staged, gate/up loads issued",
             "gate/up weights landed + dot", "act store + act wait (down rows, router rows landing)",
             "down dot", "combine + next partials written"]
    stage = {n: [] for n in names}
    stage_max = {n: [] for n in names}
    hop_part, hop_act, skew7, skew4, layer_us, launch_us = [], [], [], [], [], []
    xcd_end = np.zeros(8)
    red_in, red_out, qs_in = [], [], []
    nq = (E + 3) // 4
    for r in runs:
        launch_us.append((r[NL - 1, :, 7].max() - r[0, :, 0].min()) * us)
        for l in range(1, NL):
            t = r[l]
            for s_i, n in enumerate(names):
                d = (t[:, s_i + 1] - t[:, s_i]) * us
                stage[n].append(np.median(d))
                stage_max[n].append(d.max())
            last7 = r[l - 1, :, 7].max()
            hop_part.append(np.median((t[:, 1] - last7) * us))
            hop_act.append(np.median((t[:, 5] - t[:, 4].max()) * us))
            skew7.append((r[l - 1, :, 7].max() - r[l - 1, :, 7].min()) * us)
            skew4.append((t[:, 4].max() - t[:, 4].min()) * us)
            layer_us.append((r[l, :, 0].min() - r[l - 1, :, 0].min()) * us)
            for x in range(8):
                xcd_end[x] += (t[x::8, 7].mean() - t[:, 0].min()) * us
            # the router's two steps: reducers' column in, their sums out, everyone's sums in
            red_in.append(np.median((t[:nq, 8] - last7) * us))
            red_out.append(np.median((t[:nq, 9] - last7) * us))
            qs_in.append(np.median((t[:, 10] - t[:nq, 9].max()) * us))
    xcd_end /= len(runs) * (NL - 1)
    lines = [f"Per-layer stages of `k_decode_fused` ({G} workgroups, one per compute unit), "
             f"{'cold-routing control' if stack.cold else 'Zipf(1.1) routing'}, {len(runs)} eager launches "
             f"after {args.warmup} warmup launches; layers 1-{NL - 1} (layer 0 follows the prologue).",
             "", f"Launch: {np.mean(launch_us):.1f} us (first layer start to last layer end); "
             f"layer: {np.median(layer_us):.2f} us median.", "",
             "| stage (ends when every thread of the workgroup is past it) | median over workgroups, us | "
             "slowest workgroup, us |", "|---|---|---|"]
    for n in names:
        lines.append(f"| {n} | {np.mean(stage[n]):.2f} | {np.mean(stage_max[n]):.2f} |")
    lines += ["", "| exchange | us |", "|---|---|",
              f"| partials hop: a workgroup has every partial, after the last one was written (median) | "
              f"{np.mean(hop_part):.2f} |",
              f"| act hop + down rows: act values in, after the last act was written (median) | "
              f"{np.mean(hop_act):.2f} |",
              f"| spread of the partials writes over workgroups | {np.mean(skew7):.2f} |",
              f"| spread of the gate/up dot ends over workgroups | {np.mean(skew4):.2f} |",
              f"| router step 1: a reducer has its column of every row, after the last row was written (median) | "
              f"{np.mean(red_in):.2f} |",
              f"| router step 1: a reducer has written its sums, after the last row was written (median) | "
              f"{np.mean(red_out):.2f} |",
              f"| router step 2: a workgroup has the sums, after the last reducer wrote (median) | "
              f"{np.mean(qs_in):.2f} |", "",
              "Mean end of layer per XCD (workgroups g with g % 8 = x), us after the layer's first start: "
              + ", ".join(f"{v:.2f}" for v in xcd_end)]
    text = "\n".join(lines)
    with open(args.decode_timeline, "w") as fh:
        fh.write(text + "\n")
    log("timeline:\n" + text)
    return {"timeline": args.decode_timeline, "launch_us": round(float(np.mean(launch_us)), 2)}


def run_gemm_timeline(args, api, torch):
    """Per-item timeline of the work-list GEMM (measurement build
    libmoe_measure.so) at prefill: for several layers, one eager gate/up and
    one down launch on that layer's routing, every workgroup's clock at its
    start, plan, each item's start, first K step and K-loop end, and its end;
    summarised as markdown into args.gemm_timeline."""
    import ctypes
    lib = api.lib()
    fn = lib.moe_debug_gemm_timeline
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    T = args.tokens or 2048
    stack = BatchStack(api, torch, args.seed, T, api.MOE_PREC_F16_MFMA, decode=False)
    for _ in range(max(args.warmup, 1)):
        stack.step()
    torch.cuda.synchronize()
    tl = np.zeros((2, 1024, 100), dtype=np.uint64)
    assert fn(tl.ctypes.data, 1) == 0
    layers = list(range(0, NL, max(1, NL // max(1, min(args.steps, NL)))))[:args.steps]
    rec = {0: [], 1: []}
    for l in layers:
        stack.gateup(l)
        stack.down(l, stack.y_probe)
        torch.cuda.synchronize()
        assert fn(tl.ctypes.data, 1) == 0
        for g in (0, 1):
            rec[g].append(tl[g].astype(np.int64).copy())
    lines, summary = summarize_gemm_timeline(rec, T, layers, max(args.warmup, 1))
    text = "\n".join(lines)
    with open(args.gemm_timeline, "w") as fh:
        fh.write(text + "\n")
    log("timeline:\n" + text)
    return {"timeline": args.gemm_timeline, **summary}


def summarize_gemm_timeline(rec, T, layers, warmup):
    """Markdown lines and summary numbers of the work-list GEMM's item
    timeline: rec[0] gate/up, rec[1] down, each a list of int64 tables
    [workgroup][slot] (slots: start, plan ready, end, compute unit << 32 |
    items; then per item: start, (item, rows, K ranges, K range) word, first
    K step's barrier, K-loop end)."""
    us = 0.01  # s_memrealtime ticks at 100 MHz
    lines = [f"Work-list GEMM `k_q4_gemm` (f16 MFMA, int4 tiles staged in LDS) at prefill, {T} tokens, "
             f"Zipf(1.1) routing: one eager launch of each GEMM on the routing of layers "
             f"{', '.join(map(str, layers))}, after {warmup} warmup steps. Clock: s_memrealtime "
             "(100 MHz), thread 0 of each workgroup. An item is (expert, tile of up to 128 pair rows, N tile, "
             "K range); its row groups are its rows in 16s.", ""]
    summary = {}
    for g, name in ((0, "gate/up"), (1, "down")):
        span, plan, tail_idle, per_wg, cu_tail, n_cu = [], [], [], [], [], []
        mate_gap, mate, kl_paired, kl_alone = {}, {}, [], []
        xcd_end = np.zeros(8)
        by_mg = {}
        first_item, kloop_step = [], []
        for r in rec[g]:
            used = r[:, 0] > 0
            r = r[used]
            t0 = r[:, 0].min()
            t_end = r[:, 2].max()
            span.append((t_end - t0) * us)
            plan.append(np.median((r[:, 1] - r[:, 0]) * us))
            tail_idle.append(np.mean((t_end - r[:, 2]) * us) / ((t_end - t0) * us))
            n_items = r[:, 3] & 0xFFFFFFFF
            per_wg.append(n_items)
            # a compute unit is idle once both of its workgroups are done
            cu = r[:, 3] >> 32
            cu_end = {}
            for w in range(r.shape[0]):
                cu_end[int(cu[w])] = max(cu_end.get(int(cu[w]), 0), int(r[w, 2]))
            cu_tail.append(np.mean([(t_end - v) * us for v in cu_end.values()]) / ((t_end - t0) * us))
            n_cu.append(len(cu_end))
            # which workgroups share a compute unit, and a K loop with the other one running or done
            first = {}
            for w in range(r.shape[0]):
                c = int(cu[w])
                if c in first:
                    mate_gap[w - first[c]] = mate_gap.get(w - first[c], 0) + 1
                    mate[w], mate[first[c]] = first[c], w
                else:
                    first[c] = w
            for w in range(r.shape[0]):
                if w not in mate:
                    continue
                m_end = r[mate[w], 2]
                for j in range(int(min(n_items[w], 24))):
                    meta, b0, k1 = r[w, 5 + 4 * j], r[w, 6 + 4 * j], r[w, 7 + 4 * j]
                    if ((meta >> 16) & 0xFFFF) != 128:
                        continue
                    if k1 <= m_end:
                        kl_paired.append((k1 - b0) * us)
                    elif b0 >= m_end:
                        kl_alone.append((k1 - b0) * us)
            mate.clear()
            for x in range(8):
                xcd_end[x] += (r[x::8, 2].mean() - t0) * us
            first_item.append(np.median((r[:, 4] - r[:, 0]) * us))
            for w in range(r.shape[0]):
                n = int(min(n_items[w], 24))
                for j in range(n):
                    s0, meta, b0, k1 = r[w, 4 + 4 * j: 8 + 4 * j]
                    nxt = r[w, 4 + 4 * (j + 1)] if j + 1 < n else r[w, 2]
                    rows = int((meta >> 16) & 0xFFFF)
                    sr = int((meta >> 8) & 0xFF)
                    mg = (rows + 15) // 16
                    d = by_mg.setdefault((mg, sr), {"setup": [], "kloop": [], "tail": []})
                    d["setup"].append((b0 - s0) * us)
                    d["kloop"].append((k1 - b0) * us)
                    d["tail"].append((nxt - k1) * us)
        xcd_end /= len(rec[g])
        allw = np.concatenate(per_wg)
        n_launch = len(rec[g])
        lines += [f"## {name}", "",
                  f"Launch span (first workgroup start to last workgroup end): {np.mean(span):.1f} us mean; "
                  f"{allw.size // n_launch} workgroups; items per workgroup min {allw.min()}, median "
                  f"{np.median(allw):.0f}, max {allw.max()}.", "",
                  f"Plan (workgroup start to work list ready in LDS): {np.mean(plan):.2f} us median. "
                  f"First item's start after workgroup start: {np.mean(first_item):.2f} us median. "
                  f"Idle tail (mean over workgroups of launch end minus own end, over the span): "
                  f"{np.mean(tail_idle):.1%}; by compute unit (launch end minus the end of the later of its "
                  f"workgroups, {np.mean(n_cu):.0f} compute units): {np.mean(cu_tail):.1%}.", "",
                  "| row groups | K ranges | items | setup: item start to first K step's barrier, us | "
                  "K loop, us | after the K loop (split sum, epilogue, next item's wait), us |",
                  "|---|---|---|---|---|---|"]
        for (mg, sr) in sorted(by_mg):
            d = by_mg[(mg, sr)]
            lines.append(f"| {mg} | {sr} | {len(d['setup']) // n_launch} per launch | "
                         f"{np.median(d['setup']):.2f} | {np.median(d['kloop']):.2f} | "
                         f"{np.median(d['tail']):.2f} |")
        lines += ["", "Mean workgroup end per XCD (workgroups g with g % 8 = x), us after the launch's first "
                  "start: " + ", ".join(f"{v:.1f}" for v in xcd_end), "",
                  "Workgroups sharing a compute unit, by the difference of their indices (pairs over all "
                  "launches): " + ", ".join(f"{k}: {v}" for k, v in sorted(mate_gap.items())) + ". "
                  f"K loop of a 128-row item: {np.median(kl_paired) if kl_paired else float('nan'):.1f} us "
                  f"median while the other workgroup of its compute unit runs ({len(kl_paired)} items), "
                  f"{np.median(kl_alone) if kl_alone else float('nan'):.1f} us once it has ended "
                  f"({len(kl_alone)} items).", ""]
        summary[name] = {"span_us": round(float(np.mean(span)), 2), "plan_us": round(float(np.mean(plan)), 2),
                         "idle_tail": round(float(np.mean(tail_idle)), 4),
                         "idle_tail_cu": round(float(np.mean(cu_tail)), 4)}
    return lines, summary


# ----------------------------------------------------------------------------- batched / prefill

class BatchStack:
    """T tokens per step through the 30 layers, experts grouped by moe_permute.
    prec FP32: grouped dequant-GEMV (batched decode); F16 MFMA: grouped
    GEMM (prefill).  decode=True feeds the last layer's output back (unit-RMS
    rescale) as the next step's input; otherwise every step re-reads the same
    input tokens."""

    def __init__(self, api, torch, seed, T, prec, decode):
        self.api, self.torch, self.T, self.prec, self.decode = api, torch, T, prec, decode
        self.dm = api.dims(D, F, E, K)
        self.arena, self.stride = build_arena(torch, api, seed)
        dev = "cuda"
        self.slots = torch.arange(E, dtype=torch.int32, device=dev)
        self.router_w = [torch.from_numpy(synth.router_weight(D, E, seed, l)).to(dev) for l in range(NL)]
        self.norm_w = [torch.from_numpy(synth.norm_weight(D, seed, l)).to(dev) for l in range(NL)]
        self.bias = torch.from_numpy(np.stack([synth.zipf_bias(E, seed, l) for l in range(NL)])).to(dev)
        self.x = torch.zeros(NL + 1, T, D, dtype=torch.float32, device=dev)  # layer l: x[l] -> x[l + 1]
        self.x[0].copy_(torch.from_numpy(synth.tokens(T, D, seed, stream=7)))
        self.h = torch.empty(T, D, dtype=torch.float32, device=dev)
        self.idx = torch.zeros(NL, T, K, dtype=torch.int32, device=dev)
        self.w = torch.zeros(NL, T, K, dtype=torch.float32, device=dev)
        self.counts = torch.zeros(NL, E, dtype=torch.int32, device=dev)
        # rows padded to 16 bytes: every device pointer the library takes is 16-byte aligned
        self.offsets = torch.zeros(NL, (E + 1 + 3) // 4 * 4, dtype=torch.int32, device=dev)[:, :E + 1]
        self.sp = torch.zeros(NL, T * K, dtype=torch.int32, device=dev)
        self.pp = torch.zeros(NL, T * K, dtype=torch.int32, device=dev)
        self.act = torch.zeros(api.moe_act_bytes(T, self.dm, prec), dtype=torch.uint8, device=dev)
        self.y_probe = torch.empty(T, D, dtype=torch.float32, device=dev)
        ws = lambda c: torch.zeros(max(api.moe_workspace_size(c, T, self.dm, prec if c >= 2 else 0), 256),
                                   dtype=torch.uint8, device=dev)
        self.ws_route, self.ws_perm, self.ws_gateup, self.ws_down = ws(0), ws(1), ws(2), ws(3)

    def arena_of(self, l):
        return self.arena[l * E * self.stride:(l + 1) * E * self.stride]

    def route(self, l, stream=None):
        a = self.api
        a.moe_route(self.x[l], self.norm_w[l], EPS, self.router_w[l], self.bias[l], self.T, self.dm, self.h,
                    self.idx[l], self.w[l], self.ws_route, stream)
        a.moe_permute(self.idx[l], self.T, self.dm, self.counts[l], self.offsets[l], self.sp[l], self.pp[l],
                      self.ws_perm, stream)

    def gateup(self, l, stream=None):
        self.api.moe_expert_q4_gateup(self.h, self.idx[l], self.slots, E, self.arena_of(l), self.stride,
                                      self.offsets[l], self.sp[l], None, 0, self.T, self.dm, self.prec, self.act,
                                      self.ws_gateup, stream)

    def down(self, l, out, stream=None):
        self.api.moe_expert_q4_down_combine(self.act, self.idx[l], self.w[l], self.slots, E, self.arena_of(l),
                                            self.stride, self.offsets[l], self.sp[l], self.pp[l], self.x[l],
                                            self.T, self.dm, self.prec, out, self.ws_down, stream)

    def step(self, stream=None):
        for l in range(NL):
            self.route(l, stream)
            self.gateup(l, stream)
            self.down(l, self.x[l + 1], stream)
        if self.decode:
            self.api.moe_rms_rescale(self.x[NL], self.T, D, EPS, self.x[0], stream)


def distinct_experts(torch, stack):
    """Per layer, the number of experts with at least one routed token."""
    torch.cuda.synchronize()
    return (stack.counts > 0).sum(dim=1).cpu().numpy()


def run_batched(args, api, torch):
    T = args.tokens or 32
    prec = {"fp32": api.MOE_PREC_FP32, "f16": api.MOE_PREC_F16_MFMA}[args.batched_prec]
    stack = BatchStack(api, torch, args.seed, T, prec, decode=True)
    graph = None if args.no_graph else graph_of(torch, stack.step)
    run = (lambda n: [stack.step() for _ in range(n)]) if graph is None else \
        (lambda n: [graph.replay() for _ in range(n)])
    ms, t_wall = timed(torch, run, args.steps, args.warmup)
    tok_s = T * 1000.0 / ms
    nd = distinct_experts(torch, stack)  # routing of the last step
    per_layer = E * D * 4 + D * 4 + nd * blob_bytes()
    step_bytes = int(per_layer.sum())
    log(f"{args.steps} steps: {ms * 1000:.1f} us/step, {tok_s:.1f} tok/s, distinct experts/layer "
        f"{nd.mean():.1f}, {step_bytes / ms / 1e6:.0f} GB/s algorithmic")
    n = args.kernel_samples
    rt_us, _ = time_launch(api, torch, api.MOE_CALL_ROUTE, lambda i: stack.route(i % NL), n)
    pm_us, _ = time_launch(api, torch, api.MOE_CALL_PERMUTE, lambda i: stack.route(i % NL), n)
    gu_us, gu_med = time_launch(api, torch, api.MOE_CALL_GATEUP, lambda i: stack.gateup(i % NL), n)
    # each timed down call reads the act its own layer's gate/up just wrote (untimed): act left by
    # another layer's routing mixes block exponents within a tile and times the rare rescale path
    dn_us, _ = time_launch(api, torch, api.MOE_CALL_DOWN_COMBINE,
                           lambda i: (stack.gateup(i % NL), stack.down(i % NL, stack.y_probe)), n)
    # the sampled gate/up launches cycle over the layers: average their bytes
    layers = [i % NL for i in range(n)]
    layers = layers[2:] if n > 4 else layers
    gu_bytes = float(np.mean([nd[l] * gateup_expert_bytes() + T * D * 4 + T * K * F * 4 for l in layers]))
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    log(f"kernels (eager, mean us): route {rt_us:.2f}  permute {pm_us:.2f}  gate/up {gu_us:.2f}  down {dn_us:.2f}")
    mfma = args.batched_prec != "fp32"
    out = base_record(tok_s, args.steps, args.warmup, ms, args.batched_prec,
                      f"batched decode, {T} concurrent tokens per step, 30 routed MoE layers x 128 experts "
                      "(d=2816, f=704, top-8, int4 groups of 64), all experts resident in HBM, Zipf(1.1) routing "
                      "independent per token, expert FFN as "
                      + (f"grouped int4 GEMM on MFMA ({args.batched_prec} operands)" if mfma else
                         "grouped int4 dequant-GEMV (fp32 accumulate)"),
                      {"tokens_per_step": T, "graph": graph is not None})
    out.update({
        "distinct_experts_per_layer": round(float(nd.mean()), 2),
        "algorithmic_bytes_per_step": step_bytes,
        "algorithmic_GBps": round(step_bytes / ms / 1e6, 1),
        "hbm_frac_step": round(step_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
        "kernel_us": {"route": round(rt_us, 3), "permute": round(pm_us, 3), "gateup": round(gu_us, 3),
                      "down_combine": round(dn_us, 3)},
        "roofline": {
            "kernel": (("k_q4_small gate/up (int4 GEMM on MFMA for experts with at most 32 pairs: one item per "
                        "(expert, 64 act columns), two waves on its K halves, weights through per-wave LDS-DMA rings)"
                        if T <= 32 else "k_q4_gemm + k_q4_small gate/up (grouped int4 GEMM on MFMA)") if mfma else
                       "k_gateup grouped (int4 gate/up dequant-GEMV over experts' token groups)"),
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_of("batched_f16") if args.batched_prec == "f16" else None,
            "algorithmic_bytes_per_launch": int(gu_bytes), "avg_launch_us": round(gu_us, 3),
        },
        "wall_s_timed": round(t_wall, 3),
    })
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args.seed, T, 20.0, f"{T}-token batched decode")
    return out


def run_prefill(args, api, torch):
    T = args.tokens or 2048
    prec = {"f16": api.MOE_PREC_F16_MFMA,
            "f16direct": api.MOE_PREC_F16_MFMA_DIRECT}[args.operands]
    stack = BatchStack(api, torch, args.seed, T, prec, decode=False)
    graph = None if args.no_graph else graph_of(torch, stack.step)
    run = (lambda n: [stack.step() for _ in range(n)]) if graph is None else \
        (lambda n: [graph.replay() for _ in range(n)])
    ms, t_wall = timed(torch, run, args.steps, args.warmup)
    tok_s = T * 1000.0 / ms
    flop_gu = 2.0 * T * K * (2 * F) * D
    flop_dn = 2.0 * T * K * D * F
    step_flop = NL * (flop_gu + flop_dn)
    step_tflops = step_flop / (ms * 1e-3) / 1e12
    log(f"{args.steps} steps: {ms:.3f} ms/step, {tok_s:.0f} tok/s, expert GEMMs {step_tflops:.0f} TFLOP/s "
        f"over the step ({step_tflops / MFMA_PEAK_TFLOPS:.1%} of peak)")
    torch.cuda.synchronize()
    cnt = stack.counts.cpu().numpy()
    n = args.kernel_samples
    rt_us, _ = time_launch(api, torch, api.MOE_CALL_ROUTE, lambda i: stack.route(i % NL), n)
    pm_us, _ = time_launch(api, torch, api.MOE_CALL_PERMUTE, lambda i: stack.route(i % NL), n)
    gu_us, gu_med = time_launch(api, torch, api.MOE_CALL_GATEUP, lambda i: stack.gateup(i % NL), n)
    # each timed down call reads the act its own layer's gate/up just wrote (untimed): act left by
    # another layer's routing mixes block exponents within a tile and times the rare rescale path
    dn_us, _ = time_launch(api, torch, api.MOE_CALL_DOWN_COMBINE,
                           lambda i: (stack.gateup(i % NL), stack.down(i % NL, stack.y_probe)), n)
    achieved = flop_gu / (gu_us * 1e-6) / 1e12
    dn_tflops = flop_dn / (dn_us * 1e-6) / 1e12
    log(f"kernels (eager, mean us): route {rt_us:.1f}  permute {pm_us:.1f}  gate/up GEMM {gu_us:.1f} "
        f"({achieved:.0f} TFLOP/s)  down GEMM {dn_us:.1f} ({dn_tflops:.0f} TFLOP/s)")
    yard = gemm_yardstick(torch, int(cnt.max()))
    log(f"yardstick: torch fp16 GEMM {yard['M']} x {yard['N']} x {yard['K']} (the hottest expert's gate/up): "
        f"{yard['TFLOPs']:.0f} TFLOP/s ({yard['frac']:.1%} of peak)")
    out = base_record(tok_s, args.steps, args.warmup, ms, "fp16",
                      f"prefill, {T} tokens x 30 routed MoE layers x 128 experts (d=2816, f=704, top-8, int4 "
                      "groups of 64), Zipf(1.1) routing, expert-grouped int4 GEMM on MFMA "
                      f"({args.operands} operands, fp32 accumulate)",
                      {"tokens_per_step": T, "graph": graph is not None})
    out.update({
        "tokens_per_expert": {"max": int(cnt.max()), "median": float(np.median(cnt)), "mean": float(cnt.mean())},
        "algorithmic_flop_per_step": step_flop,
        "mfma_frac_step": round(step_tflops / MFMA_PEAK_TFLOPS, 4),
        "kernel_us": {"route": round(rt_us, 2), "permute": round(pm_us, 2), "gateup_gemm": round(gu_us, 2),
                      "down_gemm": round(dn_us, 2)},
        "roofline": {
            "kernel": f"k_q4_gemm gate/up ({args.operands} MFMA 16x16x32, int4 "
                      + ("loaded straight into registers" if args.operands == "f16direct" else "tiles staged in LDS")
                      + ", dequantised in registers)",
            "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": traffic_of("prefill"),
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated, median "
                            "over the 30 layers' launches)",
            "algorithmic_flop_per_launch": flop_gu, "avg_launch_us": round(gu_us, 2),
        },
        "wall_s_timed": round(t_wall, 3),
        "yardstick": yard,
    })
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args.seed, 256, 20.0, "prefill")
    return out


def gemm_yardstick(torch, M, reps=50):
    """Achievable-peak yardstick: a dense fp16 GEMM through torch (hipBLASLt)
    at the hottest expert's gate/up shape, M routed rows x N = 2f weight rows
    x K = d, contiguous operands, fp32 accumulate; run, never disassembled."""
    a = torch.randn(M, D, dtype=torch.float16, device="cuda")
    b = torch.randn(D, 2 * F, dtype=torch.float16, device="cuda")
    for _ in range(5):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    tf = 2.0 * M * D * 2 * F / (us * 1e-6) / 1e12
    return {"what": "torch.matmul fp16 (hipBLASLt) at the hottest expert's gate/up shape", "M": M, "N": 2 * F,
            "K": D, "us": round(us, 2), "TFLOPs": round(tf, 1), "frac": round(tf / MFMA_PEAK_TFLOPS, 4)}


# ----------------------------------------------------------------------------- bounded cache

def staging_burst(api, torch, pool, blob, stride, n_streams, steps=8, slots=64):
    """Pinned-host -> HBM staging rate of each staging mode: `steps` steps of 8
    misses each (64 distinct experts of layer 0 into an empty 64-slot layer),
    timed from the first stage call to the last copy landing."""
    res = {}
    for name, mode in (("copy", (api.MOE_STAGE_COPY, 0)), (f"split{n_streams}", (api.MOE_STAGE_COPY_SPLIT, n_streams)),
                       ("kernel", (api.MOE_STAGE_KERNEL, 0))):
        arena = torch.zeros(slots * stride, dtype=torch.uint8, device="cuda")
        tables = torch.full((1, E), -1, dtype=torch.int32, device="cuda")
        hit = torch.zeros(16, dtype=torch.uint8, device="cuda")[:K]
        side, compute = torch.cuda.Stream(), torch.cuda.current_stream()
        best = 0.0
        for rep in range(3):
            cache = api.MoeCache(1, E, slots, K, pool, blob, arena, stride, tables)
            api.moe_cache_set_staging(cache, *mode)
            sels = [torch.arange(8 * i, 8 * i + 8, dtype=torch.int32) for i in range(steps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i, sel in enumerate(sels):
                api.moe_slot_stage(cache, 0, i, sel, side, compute, hit)
            api.moe_cache_wait(cache, 0, compute)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            best = max(best, steps * 8 * blob / dt / 1e9)
            cache.close()
        # every slot holds its blob
        want = pool[:8 * steps * blob].view(8 * steps, blob)
        got = arena.view(slots, stride)[:8 * steps, :blob].cpu()
        assert torch.equal(got, want), name
        res[name] = round(best, 2)
        del arena
    return res


def policy_name(args):
    return {"lru": "LRU", "lfu": "LFU (whole-run counts)",
            "lfu-window": f"LFU ({args.lfu_window}-step window)"}[args.policy]


def run_cache(args, api, torch):
    n_slots = args.slots
    dm = api.dims(D, F, E, K)
    stride = api.moe_expert_blob_bytes(dm)
    blob = blob_bytes()
    dev = "cuda"
    total_steps = args.warmup + args.steps
    t0 = time.time()
    pool = torch.empty(NL * E * blob, dtype=torch.uint8, pin_memory=True)
    for l in range(NL):
        pool[l * E * blob:(l + 1) * E * blob].copy_(
            torch.from_numpy(np.concatenate(synth.expert_blobs(D, F, args.seed, l, range(E), threads=16))))
    log(f"pinned host pool {pool.numel() / 1e9:.2f} GB filled in {time.time() - t0:.1f} s")
    arena = torch.zeros(NL * n_slots * stride, dtype=torch.uint8, device=dev)
    tables = torch.full((NL, E), -1, dtype=torch.int32, device=dev)
    cache = api.MoeCache(NL, E, n_slots, K, pool, blob, arena, stride, tables)
    policy = {"lru": api.MOE_CACHE_LRU, "lfu": api.MOE_CACHE_LFU, "lfu-window": api.MOE_CACHE_LFU_WINDOW}[args.policy]
    api.moe_cache_set_policy(cache, policy, args.lfu_window)
    staging = {"copy": (api.MOE_STAGE_COPY, 0), "split": (api.MOE_STAGE_COPY_SPLIT, args.staging_streams),
               "kernel": (api.MOE_STAGE_KERNEL, 0)}[args.staging]
    api.moe_cache_set_staging(cache, *staging)
    on_device = args.cache_path == "device"
    if on_device:
        api.moe_cache_enable_device(cache)
    sel = np.stack([synth.markov_selections(E, K, total_steps, args.seed, l) for l in range(NL)], axis=1)
    bias = torch.from_numpy(synth.selection_bias(sel, E)).to(dev)  # [steps, NL, E]
    router_w = [torch.from_numpy(synth.router_weight(D, E, args.seed, l)).to(dev) for l in range(NL)]
    norm_w = [torch.from_numpy(synth.norm_weight(D, args.seed, l)).to(dev) for l in range(NL)]
    shared = args.overlap == "shared"
    if shared:
        # the shared expert: gated bf16 FFN of width F_SH, one copy per layer
        w_sh_gu = torch.from_numpy(synth.shared_weight_bf16(2 * F_SH, D, args.seed, 0).view(np.int16)).to(dev)
        w_sh_dn = torch.from_numpy(synth.shared_weight_bf16(D, F_SH, args.seed, 1).view(np.int16)).to(dev)
        gu_layers = w_sh_gu.unsqueeze(0).repeat(NL, 1, 1)
        dn_layers = w_sh_dn.unsqueeze(0).repeat(NL, 1, 1)
        del w_sh_gu, w_sh_dn
        res = torch.empty(1, D, dtype=torch.float32, device=dev)
        sh_ws = torch.zeros(api.moe_shared_expert_workspace_size(1, F_SH), dtype=torch.uint8, device=dev)
    else:
        w_sh = torch.from_numpy(synth.shared_weight_bf16(4 * D, D, args.seed, 0).view(np.int16)).to(dev)
        w_sh_layers = w_sh.unsqueeze(0).repeat(NL, 1, 1)  # one HBM copy per layer: no cache reuse across layers
        del w_sh
    s_out = torch.empty(1, 4 * D, dtype=torch.float32, device=dev)
    x = torch.zeros(NL + 1, 1, D, dtype=torch.float32, device=dev)
    x[0].copy_(torch.from_numpy(synth.tokens(1, D, args.seed)))
    h = torch.empty(1, D, dtype=torch.float32, device=dev)
    idx = torch.zeros(NL, 1, K, dtype=torch.int32, device=dev)
    wts = torch.zeros(NL, 1, K, dtype=torch.float32, device=dev)
    idx_host = torch.zeros(NL, K, dtype=torch.int32, pin_memory=True)
    hit_dev = torch.zeros(NL, 16, dtype=torch.uint8, device=dev)[:, :K]  # 16-byte aligned rows
    act = torch.zeros(K, F, dtype=torch.float32, device=dev)
    ws = lambda c: torch.zeros(max(api.moe_workspace_size(c, 1, dm), 256), dtype=torch.uint8, device=dev)
    ws_route, ws_gu, ws_dn = ws(0), ws(2), ws(3)
    compute = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    routed_ok = [0, 0]

    idx_all = torch.zeros(total_steps, NL, K, dtype=torch.int32, device=dev) if on_device else None

    def step(t, read_stats=True):
        stats = None
        compute = torch.cuda.current_stream()  # the capture stream while a graph is recorded
        for l in range(NL):
            a_l = arena[l * n_slots * stride:(l + 1) * n_slots * stride]
            table = tables[l]
            api.moe_route(x[l], norm_w[l], EPS, router_w[l], bias[t, l], 1, dm, h, idx[l], wts[l], ws_route)
            if on_device:
                # the rule and the miss copies on the device: no host round trip
                idx_all[t, l].copy_(idx[l, 0])
                api.moe_slot_stage_device(cache, l, t, idx[l, 0], side, compute, hit_dev[l])
            else:
                idx_host[l].copy_(idx[l, 0], non_blocking=True)
                compute.synchronize()
                routed_ok[0] += int(np.array_equal(np.sort(idx_host[l].numpy()), sel[t, l]))
                routed_ok[1] += 1
                stats = api.moe_slot_stage(cache, l, t, idx_host[l], side, compute, hit_dev[l])
            # hits first: their slots are already resident
            api.moe_expert_q4_gateup(h, idx[l], table, n_slots, a_l, stride, None, None, hit_dev[l], 1, 1, dm,
                                     api.MOE_PREC_FP32, act, ws_gu)
            # shared-path work on the compute stream while misses land: the
            # shared expert (into the combine's residual) or the filler GEMV
            if shared:
                api.moe_shared_expert_bf16(gu_layers[l], dn_layers[l], h, x[l], 1, D, F_SH, res, sh_ws)
            else:
                api.moe_shared_gemv_bf16(w_sh_layers[l], h, 1, 4 * D, D, s_out)
            api.moe_cache_wait(cache, l, compute)
            api.moe_expert_q4_gateup(h, idx[l], table, n_slots, a_l, stride, None, None, hit_dev[l], 0, 1, dm,
                                     api.MOE_PREC_FP32, act, ws_gu)
            api.moe_expert_q4_down_combine(act, idx[l], wts[l], table, n_slots, a_l, stride, None, None, None,
                                           res if shared else x[l], 1, dm, api.MOE_PREC_FP32, x[l + 1], ws_dn)
        api.moe_rms_rescale(x[NL], 1, D, EPS, x[0])
        return api.moe_cache_stats(cache) if (on_device and read_stats and t in stat_steps) else stats

    stat_steps = {args.warmup - 1, total_steps - 1}  # device mode: read the statistics back only here
    log(f"warmup {args.warmup} steps (cold cache included in the hit statistics)")
    st0 = None
    for t in range(args.warmup):
        st0 = step(t)
    torch.cuda.synchronize()
    h0, m0, b0 = (st0.hits, st0.misses, st0.bytes_staged) if st0 is not None else (0, 0, 0)
    graphs = None
    if on_device and not args.no_graph:
        # With the cache on the device a step never waits for the host, so each
        # step (its own routing bias and step number) is recorded as one HIP
        # graph before the timed region and replayed in order.
        t_cap = time.time()
        cap = torch.cuda.Stream()
        graphs = []
        for t in range(args.warmup, total_steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(t, read_stats=False)
            graphs.append(g)
        torch.cuda.synchronize()
        log(f"{len(graphs)} step graphs recorded in {time.time() - t_cap:.1f} s")
    t_wall = time.perf_counter()
    st = None
    if graphs is not None:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        st = api.moe_cache_stats(cache)
    else:
        for t in range(args.warmup, total_steps):
            st = step(t)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = t_wall * 1000.0 / args.steps
    tok_s = 1000.0 / ms
    hits, misses, staged = st.hits, st.misses, st.bytes_staged
    if on_device:  # the router's choices against the Markov selections, after the run
        got = np.sort(idx_all.cpu().numpy(), axis=-1)
        routed_ok[0] = int((got == np.sort(sel, axis=-1)).all(axis=-1).sum())
        routed_ok[1] = got.shape[0] * got.shape[1]
    th, tm, tb = hits - h0, misses - m0, staged - b0
    log(f"{args.steps} steps: {ms:.3f} ms/step, {tok_s:.1f} tok/s; hit rate {hits / (hits + misses):.4f} "
        f"(timed {th / max(1, th + tm):.4f}); {tb / args.steps / 1e6:.1f} MB staged per token")
    out = base_record(tok_s, args.steps, args.warmup, ms, "fp32",
                      f"batch-1 decode with a bounded expert cache: {n_slots} HBM slots per layer of 128 experts, "
                      f"{policy_name(args)} eviction, "
                      "expert pool in pinned host memory, misses staged on a side stream, Markov routing "
                      "(keep 0.8, Zipf refill), "
                      + (f"bf16 shared expert (gated, width {F_SH}) into the combine" if shared else
                         "bf16 shared-path GEMV (4d x d)") + " overlapped on the compute stream",
                      {"tokens_per_step": 1, "slots_per_layer": n_slots, "policy": policy_name(args),
                       "overlap": args.overlap,
                       "graph": on_device and not args.no_graph})
    out.update({
        "hit_rate": round(hits / max(1, hits + misses), 5),
        "hit_rate_timed": round(th / max(1, th + tm), 5),
        "staged_bytes_per_token": round(tb / args.steps, 1),
        "staged_GBps": round(tb / t_wall / 1e9, 2),
        "routing_matches_selection": routed_ok[0] == routed_ok[1],
        "wall_s_timed": round(t_wall, 3),
        "staging": args.staging + (str(args.staging_streams) if args.staging == "split" else ""),
        "cache_path": args.cache_path,
        "graph": graphs is not None,
    })
    cache.close()
    del arena
    out["staging_burst_GBps"] = staging_burst(api, torch, pool, blob, stride, args.staging_streams)
    log(f"staging bursts (GB/s): {out['staging_burst_GBps']}")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args.seed, 1, 20.0, "batch-1 decode (Markov routing)",
                                           bias_of=lambda l: synth.selection_bias(sel[0, l], E))
    return out


def run_cache_overlap(args, api, torch):
    """How much of the expert staging the GPU hides, and the finer overlap.

    Host cache, one hipMemcpyAsync per miss.  Three arms run the same Markov
    routing, the same kernels and the same per-layer host round trip:
      coarse    hits first, shared-path work while the misses land, one wait
                for the layer's whole staging, then the misses' gate/up;
      fine      hits first, shared-path work, then each miss's gate/up as soon
                as its own copy has landed (moe_cache_wait_expert), in the
                order the misses are copied;
      resident  every expert already in HBM (no staging at all): the time the
                step would take if staging were free.
    Each repeat runs the three arms in a rotated order (CFR, FRC, RCF, ...)
    from a fresh cache, args.repeats times; per arm the median and the spread
    are reported.  Overlap fraction = (resident + copy - arm) / copy, where
    copy = the arm's staged bytes per token at the measured burst rate of the
    same copies: 1 when staging is hidden completely, 0 when it adds its full
    time to the step."""
    n_slots = args.slots
    dm = api.dims(D, F, E, K)
    stride = api.moe_expert_blob_bytes(dm)
    blob = blob_bytes()
    dev = "cuda"
    total = args.warmup + args.steps
    t0 = time.time()
    pool = torch.empty(NL * E * blob, dtype=torch.uint8, pin_memory=True)
    for l in range(NL):
        pool[l * E * blob:(l + 1) * E * blob].copy_(
            torch.from_numpy(np.concatenate(synth.expert_blobs(D, F, args.seed, l, range(E), threads=16))))
    log(f"pinned host pool {pool.numel() / 1e9:.2f} GB filled in {time.time() - t0:.1f} s")
    sel = np.stack([synth.markov_selections(E, K, total, args.seed, l) for l in range(NL)], axis=1)
    bias = torch.from_numpy(synth.selection_bias(sel, E)).to(dev)
    router_w = [torch.from_numpy(synth.router_weight(D, E, args.seed, l)).to(dev) for l in range(NL)]
    norm_w = [torch.from_numpy(synth.norm_weight(D, args.seed, l)).to(dev) for l in range(NL)]
    w_sh = torch.from_numpy(synth.shared_weight_bf16(4 * D, D, args.seed, 0).view(np.int16)).to(dev)
    w_sh_layers = w_sh.unsqueeze(0).repeat(NL, 1, 1)
    del w_sh
    s_out = torch.empty(1, 4 * D, dtype=torch.float32, device=dev)
    x = torch.zeros(NL + 1, 1, D, dtype=torch.float32, device=dev)
    x0 = torch.from_numpy(synth.tokens(1, D, args.seed)).to(dev)
    h = torch.empty(1, D, dtype=torch.float32, device=dev)
    idx = torch.zeros(NL, 1, K, dtype=torch.int32, device=dev)
    wts = torch.zeros(NL, 1, K, dtype=torch.float32, device=dev)
    idx_host = torch.zeros(NL, K, dtype=torch.int32, pin_memory=True)
    hit_dev = torch.zeros(NL, 16, dtype=torch.uint8, device=dev)[:, :K]
    hit_host = torch.zeros(NL, K, dtype=torch.uint8)
    onehot = torch.zeros(K, 16, dtype=torch.uint8)
    for j in range(K):
        onehot[j, j] = 1
    onehot = onehot.to(dev)
    act = torch.zeros(K, F, dtype=torch.float32, device=dev)
    ws = lambda c: torch.zeros(max(api.moe_workspace_size(c, 1, dm), 256), dtype=torch.uint8, device=dev)
    ws_route, ws_gu, ws_dn = ws(0), ws(2), ws(3)
    side = torch.cuda.Stream()
    # the resident arm: all experts in HBM, identity slot tables, every pair a hit
    res_arena = torch.empty(NL * E * stride, dtype=torch.uint8, device=dev)
    res_arena.view(NL * E, stride)[:, :blob].copy_(pool.view(NL * E, blob))
    res_tables = torch.arange(E, dtype=torch.int32, device=dev).repeat(NL, 1)
    all_hit = torch.ones(16, dtype=torch.uint8, device=dev)[:K]

    def run_arm(arm):
        compute = torch.cuda.current_stream()
        if arm != "resident":
            arena = torch.zeros(NL * n_slots * stride, dtype=torch.uint8, device=dev)
            tables = torch.full((NL, E), -1, dtype=torch.int32, device=dev)
            cache = api.MoeCache(NL, E, n_slots, K, pool, blob, arena, stride, tables)
        x[0].copy_(x0)
        staged = [0]

        def step(t):
            for l in range(NL):
                api.moe_route(x[l], norm_w[l], EPS, router_w[l], bias[t, l], 1, dm, h, idx[l], wts[l], ws_route)
                idx_host[l].copy_(idx[l, 0], non_blocking=True)
                compute.synchronize()
                if arm == "resident":
                    a_l, table, hits, n_sl = res_arena[l * E * stride:(l + 1) * E * stride], res_tables[l], all_hit, E
                else:
                    a_l, table, hits, n_sl = arena[l * n_slots * stride:(l + 1) * n_slots * stride], tables[l], \
                        hit_dev[l], n_slots
                    st = api.moe_slot_stage(cache, l, t, idx_host[l], side, compute, hit_dev[l], hit_host[l])
                    staged[0] = st.bytes_staged
                api.moe_expert_q4_gateup(h, idx[l], table, n_sl, a_l, stride, None, None, hits, 1, 1, dm,
                                         api.MOE_PREC_FP32, act, ws_gu)
                api.moe_shared_gemv_bf16(w_sh_layers[l], h, 1, 4 * D, D, s_out)
                if arm == "fine":
                    misses = sorted((int(idx_host[l, j]), j) for j in range(K) if int(hit_host[l, j]) == 0)
                    for _, j in misses:
                        api.moe_cache_wait_expert(cache, l, j, compute)
                        api.moe_expert_q4_gateup(h, idx[l], table, n_sl, a_l, stride, None, None, onehot[j, :K], 1,
                                                 1, dm, api.MOE_PREC_FP32, act, ws_gu)
                else:
                    if arm == "coarse":
                        api.moe_cache_wait(cache, l, compute)
                    api.moe_expert_q4_gateup(h, idx[l], table, n_sl, a_l, stride, None, None, hits, 0, 1, dm,
                                             api.MOE_PREC_FP32, act, ws_gu)
                api.moe_expert_q4_down_combine(act, idx[l], wts[l], table, n_sl, a_l, stride, None, None, None,
                                               x[l], 1, dm, api.MOE_PREC_FP32, x[l + 1], ws_dn)
            api.moe_rms_rescale(x[NL], 1, D, EPS, x[0])

        for t in range(args.warmup):
            step(t)
        torch.cuda.synchronize()
        b0 = staged[0]
        t_wall = time.perf_counter()
        for t in range(args.warmup, total):
            step(t)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t_wall) * 1000.0 / args.steps
        y = x[NL].clone()
        if arm != "resident":
            cache.close()
            del arena
        return ms, (staged[0] - b0) / args.steps, y

    R = max(1, args.repeats)
    names = ["coarse", "fine", "resident"]
    times = {a: [] for a in names}
    staged_per_token = {}
    outs = {}
    for r in range(R):
        order = names[r % 3:] + names[:r % 3]
        for arm in order:
            ms, per_tok, y = run_arm(arm)
            times[arm].append(ms)
            staged_per_token[arm] = per_tok
            outs[arm] = y
        log(f"repeat {r}: " + ", ".join(f"{a} {times[a][-1]:.3f} ms" for a in order))
    # the three arms compute the same values: identical outputs after the last step
    same = bool(torch.equal(outs["coarse"], outs["fine"]) and torch.equal(outs["coarse"], outs["resident"]))
    burst = staging_burst(api, torch, pool, blob, stride, 2)["copy"]
    med = {a: float(np.median(times[a])) for a in names}
    copy_ms = staged_per_token["coarse"] / (burst * 1e9) * 1000.0
    raw = {a: (med["resident"] + copy_ms - med[a]) / copy_ms if copy_ms > 0 else None for a in ("coarse", "fine")}
    frac = {a: None if v is None else round(min(1.0, max(0.0, v)), 4) for a, v in raw.items()}
    log(f"medians (ms/token): coarse {med['coarse']:.3f}, fine {med['fine']:.3f}, resident {med['resident']:.3f}; "
        f"staging {staged_per_token['coarse'] / 1e6:.1f} MB/token = {copy_ms:.3f} ms at {burst:.1f} GB/s; "
        f"overlap fraction coarse {frac['coarse']}, fine {frac['fine']}; outputs identical: {same}")
    out = base_record(1000.0 / med["coarse"], args.steps, args.warmup, med["coarse"], "fp32",
                      f"batch-1 decode with a bounded expert cache: {n_slots} HBM slots per layer of 128 experts, "
                      "LRU eviction, pinned host pool, one copy per miss on a side stream, Markov routing (keep 0.8, "
                      "Zipf refill), bf16 shared-path GEMV (4d x d) on the compute stream; overlap study",
                      {"tokens_per_step": 1, "slots_per_layer": n_slots, "graph": False})
    out.update({
        "arms_ms_per_token": {a: {"median": round(med[a], 4), "min": round(min(times[a]), 4),
                                  "max": round(max(times[a]), 4), "runs": [round(v, 4) for v in times[a]]}
                              for a in names},
        "arms_tok_s_median": {a: round(1000.0 / med[a], 2) for a in names},
        "protocol": {"arms": "coarse (hits first, one wait), fine (per-miss waits), resident (no staging)",
                     "order": "rotated per repeat: CFR, FRC, RCF, ...", "repeats": R,
                     "fresh_cache_per_run": True},
        "staged_bytes_per_token": round(staged_per_token["coarse"], 1),
        "copy_burst_GBps": burst,
        "copy_ms_per_token": round(copy_ms, 4),
        "overlap_fraction": frac,
        "overlap_fraction_unclipped": {a: None if v is None else round(v, 4) for a, v in raw.items()},
        "staging_cost_ms_per_token": {a: round(med[a] - med["resident"], 4) for a in ("coarse", "fine")},
        "outputs_identical": same,
    })
    return out


def run_issue_probe(out_md):
    """Whether packed fp16 VALU work runs alongside fp16 MFMAs on one SIMD
    (measurement build): the issue probe's four modes, one workgroup of 8
    waves per compute unit, each timed 3 times (fastest kept)."""
    import ctypes
    import torch
    from int4_routed_expert_route_amd import build as moe_build
    lib = ctypes.CDLL(moe_build.MEASURE_LIB)
    fn = lib.moe_debug_issue_probe
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    groups, iters = torch.cuda.get_device_properties(0).multi_processor_count, 20000
    out = torch.zeros(groups * 512, dtype=torch.float32, device="cuda")
    names = {1: "MFMA waves only (one per SIMD: 8 MFMAs per step)",
             2: "VALU waves only (one per SIMD: 32 v_pk_fma_f16 per step)",
             3: "both at once: one MFMA wave and one VALU wave per SIMD",
             4: "mixed: every wave runs half the steps with 4 v_pk_fma_f16 after each MFMA"}
    ms = {}
    for mode in (1, 2, 3, 4):
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert fn(mode, groups, iters, out.data_ptr(), None) == 0
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        ms[mode] = best
    lines = [f"Issue probe (`k_issue_probe`, measurement build): {groups} workgroups of 8 waves (one per compute "
             f"unit, two waves per SIMD), {iters} steps per working wave; fastest of 3 launches.", "",
             "| mode | ms | us per step |", "|---|---|---|"]
    for mode in (1, 2, 3, 4):
        lines.append(f"| {names[mode]} | {ms[mode]:.3f} | {ms[mode] * 1e3 / iters:.4f} |")
    lines += ["", f"Sum of the MFMA-only and VALU-only times: {ms[1] + ms[2]:.3f} ms; the longer of the two: "
              f"{max(ms[1], ms[2]):.3f} ms. Both at once took {ms[3]:.3f} ms and mixed {ms[4]:.3f} ms, so "
              f"{(ms[1] + ms[2] - ms[3]) / min(ms[1], ms[2]):.0%} (separate waves) and "
              f"{(ms[1] + ms[2] - ms[4]) / min(ms[1], ms[2]):.0%} (mixed in each wave) of the shorter part was "
              "hidden under the longer."]
    text = "\n".join(lines)
    with open(out_md, "w") as fh:
        fh.write(text + "\n")
    log("issue probe:\n" + text)
    print(json.dumps({"issue_probe": out_md, "ms": ms}), flush=True)


def run_copy_calibration(mib):
    """Known-bytes kernels for scaling HBM counters: a device-to-device copy of
    MIB MiB (torch), and, from the measurement build, reads of the same bytes
    with 128-bit loads into registers and with LDS-DMA loads (three launches
    each, on buffers larger than the last-level cache)."""
    import ctypes
    import torch
    from int4_routed_expert_route_amd import build as moe_build
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    rec = {"copy_bytes_per_launch": n, "launches": 3}
    if os.path.exists(moe_build.MEASURE_LIB):
        lib = ctypes.CDLL(moe_build.MEASURE_LIB)
        fn = lib.moe_debug_read
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        out = torch.zeros(1024 * 256, dtype=torch.int32, device="cuda")
        for mode in (0, 1):
            for _ in range(3):
                assert fn(src.data_ptr(), n, mode, out.data_ptr(), None) == 0
        torch.cuda.synchronize()
        rec.update({"read_bytes_per_launch": n, "read_modes": ["vgpr_b128", "lds_dma_16B"]})
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", choices=["decode", "batched", "prefill", "cache"], default="decode")
    ap.add_argument("--control", choices=["zipf", "cold"], default="zipf",
                    help="--decode-timeline: zipf = the Zipf(1.1) routing workload; cold = routing that never "
                         "reuses an expert within 16 steps (defeats the last-level cache).  The decode timing "
                         "line always runs both, alternated")
    ap.add_argument("--tokens", type=int, default=0, help="batched / prefill: tokens per step (32 / 2048)")
    ap.add_argument("--decode-path", choices=["fused", "calls"], default="fused",
                    help="decode: one moe_decode_layers launch per token, or the three calls per layer")
    ap.add_argument("--operands", choices=["f16", "f16direct"], default="f16",
                    help="prefill: MFMA operand type (f16direct: fp16 with int4 weights loaded straight into "
                         "registers, the ablation of the staged tile)")
    ap.add_argument("--batched-prec", choices=["fp32", "f16"], default="f16",
                    help="batched: fp32 dequant-GEMV or grouped GEMM on MFMA")
    ap.add_argument("--slots", type=int, default=64, help="cache: HBM slots per layer")
    ap.add_argument("--policy", choices=["lru", "lfu", "lfu-window"], default="lru", help="cache: eviction policy")
    ap.add_argument("--lfu-window", type=int, default=64, help="cache: steps counted by --policy lfu-window")
    ap.add_argument("--staging", choices=["copy", "split", "kernel"], default="copy",
                    help="cache: how misses are copied (one DMA copy, split over streams, device-pulled kernel)")
    ap.add_argument("--staging-streams", type=int, default=4, help="cache: streams for --staging split")
    ap.add_argument("--cache-path", choices=["host", "device"], default="host",
                    help="cache: eviction rule and miss copies on the host (one sync per layer) or on the device")
    ap.add_argument("--overlap", choices=["filler", "shared"], default="filler",
                    help="cache: work overlapped with staging (the d x 4d filler GEMV, or the shared expert)")
    ap.add_argument("--overlap-study", action="store_true",
                    help="cache: coarse, fine (per-miss) and resident arms alternated, with the overlap fraction")
    ap.add_argument("--kernel-samples", type=int, default=62)
    ap.add_argument("--repeats", type=int, default=5,
                    help="decode: timed segments per arm (Zipf workload and cold-routing control, alternated)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--decode-timeline", default="", metavar="OUT.md",
                    help="decode: per-stage timeline of the fused kernel from the measurement build "
                         "libmoe_measure.so, summarised into OUT.md (no timing line)")
    ap.add_argument("--gemm-timeline", default="", metavar="OUT.md",
                    help="prefill: per-item timeline of the work-list GEMM from the measurement build "
                         "libmoe_measure.so over --steps layers, summarised into OUT.md (no timing line)")
    ap.add_argument("--issue-probe", default="", metavar="OUT.md",
                    help="only run the MFMA / packed-fp16 VALU issue probe of the measurement build, into OUT.md")
    ap.add_argument("--library", default="", metavar="SO",
                    help="load this build of libmoe instead of the in-tree one (compare builds on one box)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling HBM counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        run_copy_calibration(args.copy_calibration)
        return
    if args.issue_probe:
        run_issue_probe(args.issue_probe)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the routed MoE hot path is built and "
                                   "measured on a single MI355X (multi-GPU expert parallelism is design-only)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    defaults = {"decode": (256, 16), "batched": (64, 4), "prefill": (10, 2), "cache": (448, 64)}
    ds, dw = defaults[args.workload]
    args.steps = ds if args.steps is None else args.steps
    args.warmup = dw if args.warmup is None else args.warmup

    import torch
    import int4_routed_expert_route_amd.api as api
    if args.decode_timeline or args.gemm_timeline:
        from int4_routed_expert_route_amd import build as moe_build
        api.LIB_PATH = moe_build.MEASURE_LIB
    if args.decode_timeline:
        args.workload = "decode"
        args.warmup, args.steps = min(args.warmup, 16), min(args.steps, 8)
    if args.gemm_timeline:
        args.workload = "prefill"
        args.warmup, args.steps = min(args.warmup, 2), min(args.steps, 6)
    if args.library:
        api.LIB_PATH = os.path.abspath(args.library)
    api.lib()
    torch.cuda.set_device(0)
    run = {"decode": run_decode, "batched": run_batched, "prefill": run_prefill, "cache": run_cache}[args.workload]
    if args.decode_timeline:
        run = run_decode_timeline
    if args.gemm_timeline:
        run = run_gemm_timeline
    if args.overlap_study:
        if args.workload != "cache":
            raise SystemExit("--overlap-study belongs to --workload cache")
        run = run_cache_overlap
    print(json.dumps(run(args, api, torch)), flush=True)


if __name__ == "__main__":
    main()
