#!/usr/bin/env python3
"""Benchmark of the routed int4 MoE hot path on one MI355X.

Default workload: batch-1 decode through a 30-layer stack of the routed MoE
layer (d=2816, f=704, 128 experts, top-8, int4 groups of 64 with fp16
scale/bias), all 3,840 experts resident in HBM slots (12.85 GB), Zipf(1.1)
expert popularity per layer.  One step = one token through all 30 layers:
per layer route -> gate/up -> down+combine, then the unit-RMS feedback to the
next step.  The step is captured once as a HIP graph and replayed.

Prints one JSON line.  `value` is tokens/s; the `roofline` object covers the
dominant kernel (gate/up dequant-GEMV), timed with HIP events at the kernel's
own begin/end on its stream; `cpu_baseline` is the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

D, F, E, K, NL = synth.D_MODEL, synth.D_FF, synth.N_EXPERTS, synth.TOP_K, synth.N_LAYERS
METRIC = "routed-MoE tokens/s + achieved HBM GB/s (int4 decode), MFMA util (prefill)"
HBM_PEAK_GBPS = 8000.0
EPS = 1e-6

# HBM bytes per gate/up launch measured with rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (scaled by a 256 MiB copy's readings), for the kernel source with
# this fingerprint; reported as null once the source differs.
GATEUP_TRAFFIC = {"source_sha256_16": "c35bc92e4b26bf04", "fetch_bytes": 18126218, "write_bytes": 22528}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes():
    """Bytes one decode token must read: per layer the router (fp32 E x d), the
    RMSNorm weight and the 8 selected expert blobs."""
    blob = 3 * D * F // 2 + 3 * D * F // 64 * 4
    per_layer = E * D * 4 + D * 4 + K * blob
    gateup_launch = K * (2 * F * D // 2 + 2 * F * (D // 64) * 4) + D * 4 + K * F * 4
    down_launch = K * (D * F // 2 + D * (F // 64) * 4) + K * F * 4 + K * 4 + 2 * D * 4
    return blob, per_layer, gateup_launch, down_launch


class DecodeStack:
    """Device state of the 30-layer decode workload."""

    def __init__(self, api, torch, seed=0, cold=False):
        self.api, self.torch = api, torch
        self.dm = api.dims(D, F, E, K)
        self.stride = api.moe_expert_blob_bytes(self.dm)
        dev = "cuda"
        t0 = time.time()
        self.arena = torch.empty(NL * E * self.stride, dtype=torch.uint8, device=dev)
        for l in range(NL):
            blobs = synth.expert_blobs(D, F, seed, l, range(E), threads=16)
            host = torch.from_numpy(np.concatenate(blobs))
            self.arena[l * E * self.stride:(l + 1) * E * self.stride].copy_(host)
        torch.cuda.synchronize()
        log(f"arena {self.arena.numel() / 1e9:.2f} GB filled in {time.time() - t0:.1f} s")
        self.slots = torch.arange(E, dtype=torch.int32, device=dev)
        self.router_w = [torch.from_numpy(synth.router_weight(D, E, seed, l)).to(dev) for l in range(NL)]
        self.norm_w = [torch.from_numpy(synth.norm_weight(D, seed, l)).to(dev) for l in range(NL)]
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
        ws = lambda c: torch.zeros(max(api.moe_workspace_size(c, 1, self.dm), 256), dtype=torch.uint8, device=dev)
        self.ws_route, self.ws_gateup, self.ws_down = ws(0), ws(2), ws(3)

    def arena_of(self, l):
        return self.arena[l * E * self.stride:(l + 1) * E * self.stride]

    def layer(self, s, l, stream=None):
        a, dm = self.api, self.dm
        a.moe_route(self.x[l:l + 1], self.norm_w[l], EPS, self.router_w[l], self.bias[s, l], 1, dm, self.h,
                    self.idx[s, l:l + 1], self.w[s, l:l + 1], self.ws_route, stream)
        a.moe_expert_q4_gateup(self.h, self.idx[s, l:l + 1], self.slots, E, self.arena_of(l), self.stride, None,
                               None, None, 0, 1, dm, a.MOE_PREC_FP32, self.act, self.ws_gateup, stream)
        a.moe_expert_q4_down_combine(self.act, self.idx[s, l:l + 1], self.w[s, l:l + 1], self.slots, E,
                                     self.arena_of(l), self.stride, None, None, None, self.x[l:l + 1], 1, dm,
                                     a.MOE_PREC_FP32, self.x[l + 1:l + 2], self.ws_down, stream)

    def steps(self, n_periods=1, stream=None):
        for _ in range(n_periods):
            for s in range(self.period):
                for l in range(NL):
                    self.layer(s, l, stream)
                self.api.moe_rms_rescale(self.x[NL:NL + 1], 1, D, EPS, self.x[0:1], stream)


def time_kernel(api, torch, stack, call, n):
    """Average duration (us) of one call's main kernel over n eager launches,
    cycling through layers, with events recorded at the kernel's own begin/end."""
    durs = []
    for i in range(n):
        l = i % NL
        s = (i // NL) % stack.period
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        api.moe_profile_next_launch(call, e0, e1)
        a, dm = api, stack.dm
        if call == api.MOE_CALL_ROUTE:
            a.moe_route(stack.x[l:l + 1], stack.norm_w[l], EPS, stack.router_w[l], stack.bias[s, l], 1, dm, stack.h,
                        stack.idx[s, l:l + 1], stack.w[s, l:l + 1], stack.ws_route)
        elif call == api.MOE_CALL_GATEUP:
            a.moe_expert_q4_gateup(stack.h, stack.idx[s, l:l + 1], stack.slots, E, stack.arena_of(l), stack.stride,
                                   None, None, None, 0, 1, dm, a.MOE_PREC_FP32, stack.act, stack.ws_gateup)
        else:
            out = torch.empty(1, D, device="cuda")
            a.moe_expert_q4_down_combine(stack.act, stack.idx[s, l:l + 1], stack.w[s, l:l + 1], stack.slots, E,
                                         stack.arena_of(l), stack.stride, None, None, None, stack.x[l:l + 1], 1,
                                         dm, a.MOE_PREC_FP32, out, stack.ws_down)
        e1.synchronize()
        durs.append(e0.elapsed_time(e1) * 1000.0)
    durs = np.array(durs[2:] if len(durs) > 4 else durs)
    return float(np.mean(durs)), float(np.median(durs))


def cpu_baseline(seed, budget_s=20.0):
    """The CPU oracle on a bounded sample of the same workload: the layers of
    one batch-1 decode step, in order, until ~budget_s of oracle time (at most
    all 30); expert blob generation is untimed.  Scaled to tokens/s of the
    30-layer stack."""
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    x = synth.tokens(1, D, seed).astype(np.float64)
    spent, done = 0.0, 0
    for l in range(NL):
        blobs = dict(zip(range(E), synth.expert_blobs(D, F, seed, l, range(E), threads=16)))
        rw = synth.router_weight(D, E, seed, l)
        nw = synth.norm_weight(D, seed, l)
        bias = synth.zipf_bias(E, seed, l)
        t0 = time.perf_counter()
        x, *_ = orc.moe_layer(x, nw, rw, bias, blobs.__getitem__, D, F, K)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    per_token = spent / done * NL
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layers 0-{done - 1} of one batch-1 decode step (Zipf routing), {spent:.1f} s of oracle "
                      f"time" + ("" if done == NL else f", scaled x{NL / done:.2f} to the 30-layer token")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--control", choices=["zipf", "cold"], default="zipf",
                    help="zipf: the Zipf(1.1) routing workload; cold: routing that never reuses an expert "
                         "within 16 steps (defeats the last-level cache)")
    ap.add_argument("--kernel-samples", type=int, default=62)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling HBM counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the routed MoE hot path is built and "
                                   "measured on a single MI355X (multi-GPU expert parallelism is design-only)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import int4_routed_expert_route_amd.api as api
    api.lib()
    torch.cuda.set_device(0)
    stack = DecodeStack(api, torch, args.seed, cold=args.control == "cold")
    period = stack.period
    steps = max(period, (args.steps + period - 1) // period * period)
    warm = max(period, (args.warmup + period - 1) // period * period)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if args.no_graph:
        run = lambda n: stack.steps(n // period)
    else:
        # one replay = one routing period (1 step for Zipf, 16 for the cold arm)
        with torch.cuda.stream(stream):
            stack.steps(1)  # eager warm-up on the capture stream
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            stack.steps(1)
        torch.cuda.synchronize()
        run = lambda n: [graph.replay() for _ in range(n // period)]
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
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / steps
    tok_s = 1000.0 / ms
    blob, per_layer, gu_bytes, down_bytes = algorithmic_bytes()
    step_bytes = NL * per_layer
    log(f"{steps} steps: {ms * 1000:.1f} us/step, {tok_s:.1f} tok/s, {step_bytes * tok_s / 1e9:.0f} GB/s algorithmic")

    # dominant kernel: gate/up dequant-GEMV, timed at its own begin/end
    gu_us, gu_med = time_kernel(api, torch, stack, api.MOE_CALL_GATEUP, args.kernel_samples)
    dn_us, _ = time_kernel(api, torch, stack, api.MOE_CALL_DOWN_COMBINE, args.kernel_samples)
    rt_us, _ = time_kernel(api, torch, stack, api.MOE_CALL_ROUTE, args.kernel_samples)
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    traffic = None
    try:
        import hashlib
        src = b"".join(open(os.path.join(ROOT, "int4_routed_expert_route_amd", "csrc", n), "rb").read()
                       for n in ("q4_gemv.hip", "common.h"))
        if hashlib.sha256(src).hexdigest()[:16] == GATEUP_TRAFFIC["source_sha256_16"]:
            traffic = GATEUP_TRAFFIC["fetch_bytes"] + GATEUP_TRAFFIC["write_bytes"]
    except OSError:
        pass
    log(f"kernels (eager, mean us): route {rt_us:.2f}  gate/up {gu_us:.2f} (median {gu_med:.2f})  down {dn_us:.2f}")

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "batch-1 decode, 30 routed MoE layers x 128 experts (d=2816, f=704, top-8, int4 "
                        "groups of 64, fp16 scale/bias), all experts resident in HBM, "
                        + ("Zipf(1.1) routing" if not stack.cold else "cold routing control (no expert reuse "
                                                                           "within 16 steps)"),
            "tokens_per_step": 1,
            "layers": NL,
            "graph": not args.no_graph,
        },
        "algorithmic_bytes_per_token": step_bytes,
        "algorithmic_GBps": round(step_bytes * tok_s / 1e9, 1),
        "hbm_frac_step": round(step_bytes * tok_s / 1e9 / HBM_PEAK_GBPS, 4),
        "kernel_us": {"route": round(rt_us, 3), "gateup": round(gu_us, 3), "down_combine": round(dn_us, 3)},
        "roofline": {
            "kernel": "k_gateup_fp32 (int4 gate/up dequant-GEMV, 8 experts)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_us, 3),
        },
        "wall_s_timed": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
