#!/usr/bin/env python3
"""Benchmark of the routed SwiGLU MoE layer on one MI355X.

One step = the whole hot path over one batch: routing + sort by expert,
forward (gate/up GEMM + SwiGLU over the routed rows gathered in its loads,
down GEMM, weighted combine) and backward (dA GEMM, recompute + SwiGLU
backward, dX GEMM, dW GEMMs, all gathering x / dy rows in their loads; dX and
dRouterWeights reductions), all through the C ABI on device-resident
inputs.  Workload: the Qwen3-30B-A3B layer shape (T=8192 tokens, D=2048,
I=768, E=128 experts, top-8, softmax-renormalised routing), synthetic seeded
inputs.

value = counted FLOPs per step / step time, with 6*D*I FLOPs per routed row
forward and 12*D*I backward (the activation recompute is not counted).

Prints ONE JSON line.  Also reports the dominant kernel against its roofline
(its duration from HIP events on its launch stream over the timed steps, in
which no other kernel carries events; the per-kernel table comes from K
instrumented steps before them) and the CPU oracle timed on a bounded sample
of the same workload.
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

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "MoE layer TFLOP/s fwd & bwd, Qwen3-30B-A3B shape, 8192 tokens, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak (no sparsity)
PEAK_FP32_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
PEAK_HBM_GBPS = 8000.0

WORKLOADS = {"qwen3_30b_a3b": synth.QWEN3_30B_A3B, "llama4_scout": synth.LLAMA4_SCOUT,
             "tiny": synth.TINY,
             # the Qwen shape with Zipf(1.2)-skewed routing over the token counts of a sweep
             **{f"qwen3_30b_a3b_zipf_T{T}": synth.qwen_zipf(T) for T in synth.ZIPF_SWEEP_T}}


def kernel_work(wl: synth.Workload) -> dict:
    """Algorithmic work per launch: ('mfma', FLOPs) for GEMMs, ('hbm', bytes) for the rest."""
    T, D, I, E, K, R = wl.T, wl.D, wl.I, wl.E, wl.K, wl.R
    dir_ = float(D) * I * R
    return {
        "gemm_gateup_h": ("mfma", 4 * dir_), "gemm_gateup_gu": ("mfma", 4 * dir_),
        "gemm_down": ("mfma", 2 * dir_), "gemm_da": ("mfma", 2 * dir_),
        # dXs (4 D I R), dW_down (2 D I R) and dW_gate + dW_up (4 D I R) in one launch
        "gemm_bwd_fused": ("mfma", 10 * dir_),
        # chained launches (many m-tiles): gate/up + down, dA + the recompute
        "gemm_fwd_chain": ("mfma", 6 * dir_), "gemm_da_recompute": ("mfma", 6 * dir_),
        # combine: read O (R*D*2), weights and indices (8R), write y (T*D*2)
        "combine": ("hbm", 2.0 * R * D + 8 * R + 2.0 * T * D),
        # dX reduce: read the fp16 per-row partials (R*D*2), write dX (T*D*2); in the
        # same launch dRouterWeights: read the per-row partials (one per gate/up column
        # tile and wave column, 4 * ceil(I / 128) per row) and the indices, write one
        # value per row
        "reduce_rows": ("hbm", 2.0 * R * D + 2.0 * T * D
                        + 4.0 * R * (4 * math.ceil(I / 128)) + 8 * R),
        "route_topk": ("hbm", 4.0 * T * E + 8 * R),
        "route_hist": ("hbm", 4.0 * R),
        # scatter: read the ids (4R) and the histogram table once, write both permutations (8R)
        "route_scatter": ("hbm", 12.0 * R + 4.0 * E * math.ceil(R / route_chunk(R))),
        "tilemap": ("hbm", 8.0 * E),
        # backward set-up: split flags from the sorted-row indices and their router
        # weights (8R), the row offsets (write 4R; the indices again from L2),
        # offsets, flags, tile starts and chunk map
        "bwd_setup": ("hbm", 12.0 * R + 24.0 * E),
        # max |dy| for the gradient scale: read dy once
        "dy_amax": ("hbm", 2.0 * T * D + 4.0 * 1024),
        # fp16 copies of x and s dy for the dW GEMMs: read both, write both
        "f16_operands": ("hbm", 8.0 * T * D),
        # router projection and router backward (timed beside the step, not in it)
        "router_logits": ("mfma32", 2.0 * T * D * E), "router_dwr": ("mfma32", 2.0 * T * D * E),
        # dX += dl W_r^T: read and write dX (4*T*D), dl and indices (8R); W_r^T rows from L2
        "router_dx": ("hbm", 4.0 * T * D + 8 * R),
        "router_dwr_sum": ("hbm", 4.0 * D * E * (router_splits(T) + 1)),
    }


def gemm_min_bytes(wl: synth.Workload) -> dict:
    """Unavoidable HBM bytes per launch of each grouped GEMM kernel with this
    dataflow: every operand read once and every result written once (the
    routed rows of x and dy count once per token, the gathers being folded into
    the loads).  With the kernel's algorithmic FLOPs this gives its
    arithmetic intensity and its attainable roof min(MFMA peak, AI x HBM)."""
    T, D, I, E, R = wl.T, wl.D, wl.I, wl.E, wl.R
    w1 = 2.0 * E * I * D  # one expert weight set, bf16
    b = {
        # x rows, W_gate + W_up, H (fp16)
        "gemm_gateup_h": 2.0 * T * D + 2 * w1 + 2.0 * R * I,
        # x rows, W_gate + W_up, dA (fp32) in; dG | dU, Hw (fp16) and the dRW partials out
        "gemm_gateup_gu": 2.0 * T * D + 2 * w1 + 4.0 * R * I + 6.0 * R * I
                          + 4.0 * R * 4 * math.ceil(I / 128),
        # H (fp16), W_down in; O (bf16) out
        "gemm_down": 2.0 * R * I + w1 + 2.0 * R * D,
        # dy rows, W_down in; dA (fp32) out
        "gemm_da": 2.0 * T * D + w1 + 4.0 * R * I,
        # dXs: dG | dU, W_gate + W_up in, fp16 dX rows out; dW_down: s dy (fp16), Hw in,
        # fp32 dW_down out; dW_gate / dW_up: x (fp16) in, fp32 dW_gate, dW_up out
        "gemm_bwd_fused": 4.0 * R * I + 2 * w1 + 2.0 * R * D + 2.0 * T * D + 2.0 * R * I
                          + 2 * w1 + 2.0 * T * D + 4 * w1,
    }
    # the chained launches move what their two GEMMs move
    b["gemm_fwd_chain"] = b["gemm_gateup_h"] + b["gemm_down"]
    b["gemm_da_recompute"] = b["gemm_da"] + b["gemm_gateup_gu"]
    return b


def route_chunk(R: int) -> int:
    """Flat slots per routing block (as the library chooses them)."""
    per = (R + 255) // 256
    per = (per + 63) // 64 * 64
    return max(1024, per)


def router_splits(T: int) -> int:
    """Token ranges of the dW_r partials (as the library chooses them)."""
    tc = max(512, (-(-T // 64) + 31) // 32 * 32)
    return max(1, -(-T // tc))


GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_expert_amd", "csrc", "gemm.hip")


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary profiles/<kernel>_<workload>_traffic.txt (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated), or None when there is none or when the GEMM source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if kv.get("gemm_source_sha256") != sha or "bytes_per_launch" not in kv:
        return None
    return float(kv["bytes_per_launch"])


def cpu_baseline(wl: synth.Workload, data: dict, n_tokens: int) -> dict:
    """The CPU oracle, as it stands, on the first n_tokens tokens of the workload:
    forward, backward (dX, dRouterWeights) and the weight gradients over those
    tokens.  Value in the metric's unit, counted with the same FLOP formula."""
    import oracle
    f = synth.bf16_bits_to_f64
    L = oracle.Layer(f(data["x"]), f(data["w_gate"]), f(data["w_up"]), f(data["w_down"]),
                     wl.K, wl.score, f(data["dy"]))
    idx, w = oracle.route(data["logits"], wl.K, wl.score)
    tok = np.arange(n_tokens, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.forward(L, idx, w, tokens=tok)
    t1 = time.perf_counter()
    oracle.backward_tokens(L, idx, w, tokens=tok)
    oracle.backward_dw(L, idx, w, tokens=tok)
    t2 = time.perf_counter()
    rows = n_tokens * wl.K
    flops = 18.0 * wl.D * wl.I * rows
    threads = oracle.threads()
    host = host_cpu()
    return {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", **host,
            "sample": (f"first {n_tokens} tokens ({rows} routed rows) of the {wl.name} workload: "
                       f"oracle forward {t1 - t0:.2f} s + backward incl. weight gradients "
                       f"{t2 - t1:.2f} s, float64, {threads} OpenMP threads on "
                       f"{host['cpu_model']}")}


def host_cpu() -> dict:
    """The host CPU: model string, logical CPUs of the machine and of this process."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": usable, "cpus_on_host": os.cpu_count() or usable}


def step_stats(step_ms: list) -> dict:
    """Median, 10th and 90th percentile and spread of per-step times (ms)."""
    a = np.sort(np.asarray(step_ms, dtype=np.float64))
    return {"median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4),
            "min": round(float(a[0]), 4), "max": round(float(a[-1]), 4), "n": int(a.size)}


def run_processes(args) -> int:
    """The measurement in args.processes fresh child processes (this process
    touches no GPU); prints the median child's line with every child's value
    and step time, then the CPU baseline measured here."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--processes", "1", "--cpu-tokens", "0",
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--workload", args.workload]
    if args.fwd_bwd_only:
        cmd.append("--fwd-bwd-only")
    lines = []
    for i in range(args.processes):
        print(f"bench: process {i + 1} of {args.processes}", file=sys.stderr, flush=True)
        res = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        if res.returncode != 0:
            print(f"bench: process {i + 1} failed with status {res.returncode}", file=sys.stderr)
            return res.returncode
        lines.append(json.loads(res.stdout.strip().splitlines()[-1]))
    order = sorted(range(len(lines)), key=lambda i: lines[i]["value"])
    out = lines[order[len(order) // 2]]
    out["processes"] = {"n": len(lines), "values": [l["value"] for l in lines],
                        "ms_per_step": [l["ms_per_step"] for l in lines],
                        "step_ms_median": [l["step_ms"]["median"] for l in lines]}
    if args.cpu_tokens > 0:
        wl = WORKLOADS[args.workload]
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, synth.generate(wl), args.cpu_tokens)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b_a3b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-tokens", type=int, default=640,
                    help="tokens in the CPU-oracle baseline sample (0: skip)")
    ap.add_argument("--fwd-bwd-only", action="store_true",
                    help="time only the full steps (skip the separate fwd/bwd timing)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="before the steps, run a plain device copy of this many MiB (twice), "
                         "as the reference dispatch that scales HBM byte counters")
    ap.add_argument("--processes", type=int, default=1,
                    help="run the GPU measurement in this many fresh processes, one after the "
                         "other, and report the one with the median value (with all values)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no sharding or collectives).", file=sys.stderr)
        return 2
    if args.processes > 1:
        return run_processes(args)

    import torch
    import mixture_experts_layer_expert_amd as moe
    from tests import gpu_common as G

    moe.load_library()
    if args.copy_calib_mb > 0:
        n = args.copy_calib_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = WORKLOADS[args.workload]
    data = synth.generate(wl)
    dev = G.DeviceInputs(data)
    d = moe.dims(wl.T, wl.D, wl.I, wl.E, wl.K, wl.score)
    ws = [torch.empty(moe.moe_workspace_bytes(d, ph), dtype=torch.uint8, device="cuda")
          for ph in range(3)]
    route = moe.moe_route_sort(dev.logits, wl.K, wl.score, ws=ws[0])
    y = torch.empty((wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    grads = moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, wl.K, wl.score,
                        ws=ws[2])
    stream = torch.cuda.current_stream()

    def step(do_route=True, do_fwd=True, do_bwd=True):
        if do_route:
            moe.moe_route_sort(dev.logits, wl.K, wl.score, out=route, ws=ws[0])
        if do_fwd:
            moe.moe_fwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, wl.K, wl.score, y=y, ws=ws[1])
        if do_bwd:
            moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, wl.K, wl.score,
                        out=grads, ws=ws[2])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: {wl.name} warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # per-kernel durations: K instrumented steps, every kernel bracketed by two
    # HIP events on its launch stream (they add ~4% to a step, so this pass is
    # not the timed region)
    work = kernel_work(wl)
    moe.moe_prof_only(None)
    moe.moe_prof_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = moe.moe_prof_read()
    moe.moe_prof_enable(False)
    gemms = {k: v for k, v in kern.items() if work.get(k, ("", 0))[0] == "mfma"}
    dom = max(gemms, key=lambda k: gemms[k][0])

    # timed region: K full steps; only the dominant kernel is bracketed by HIP
    # events (on its launch stream), for its live average duration, and an
    # event on the launch stream marks every step boundary (per-step times)
    moe.moe_prof_only(dom)
    moe.moe_prof_enable(True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    dom_ms, dom_n = moe.moe_prof_read()[dom]
    moe.moe_prof_enable(False)
    moe.moe_prof_only(None)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flops_step = wl.flops_fwd() + wl.flops_bwd()
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # forward-only and backward-only rates (event-timed on the same stream)
    extra = {}
    if not args.fwd_bwd_only:
        for name, kw in (("fwd", dict(do_route=False, do_bwd=False)),
                         ("bwd", dict(do_route=False, do_fwd=False))):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(args.steps):
                step(**kw)
            ev1.record(stream)
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / args.steps
            fl = wl.flops_fwd() if name == "fwd" else wl.flops_bwd()
            extra[f"{name}_ms"] = round(ms, 4)
            extra[f"{name}_tflops"] = round(fl / (ms * 1e-3) / 1e12, 2)

    # router projection + router backward, timed on their own (not part of the step)
    router = None
    if not args.fwd_bwd_only:
        w_r = G.to_dev(data["w_r"])
        logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device="cuda")
        ws_r = torch.empty(moe.moe_workspace_bytes(d, moe.MOE_PHASE_ROUTER_BWD), dtype=torch.uint8,
                           device="cuda")
        dx_r = grads["dx"].clone()
        dw_r = torch.empty((wl.D, wl.E), dtype=torch.float32, device="cuda")

        def rstep(fwd=True, bwd=True):
            if fwd:
                moe.moe_router_fwd(dev.x, w_r, logits=logits)
            if bwd:
                moe.moe_router_bwd(dev.x, w_r, route, grads["d_topk_w"], dx_r, wl.K, wl.score,
                                   dw_r=dw_r, ws=ws_r)

        for _ in range(args.warmup):
            rstep()
        torch.cuda.synchronize()
        moe.moe_prof_enable(True)
        router = {}
        for name, kw in (("fwd", dict(bwd=False)), ("bwd", dict(fwd=False))):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(args.steps):
                rstep(**kw)
            ev1.record(stream)
            torch.cuda.synchronize()
            router[f"{name}_ms"] = round(ev0.elapsed_time(ev1) / args.steps, 4)
        kern.update(moe.moe_prof_read())
        moe.moe_prof_enable(False)

    kernels = {}
    min_bytes = gemm_min_bytes(wl)

    def ceiling_tflops(name):
        # attainable roof of a GEMM: min(MFMA peak, arithmetic intensity x HBM)
        return min(PEAK_BF16_TFLOPS, work[name][1] / min_bytes[name] * PEAK_HBM_GBPS / 1e3)

    for name, (tot_ms, n) in kern.items():
        avg_ms = tot_ms / n
        bound, amount = work.get(name, ("hbm", 0.0))
        rate = amount / (avg_ms * 1e-3)
        if bound in ("mfma", "mfma32"):
            peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_FP32_TFLOPS
            kernels[name] = {"avg_us": round(avg_ms * 1e3, 2), "launches": n, "bound": bound,
                             "tflops": round(rate / 1e12, 2), "frac": round(rate / 1e12 / peak, 4)}
            if name in min_bytes:
                c = ceiling_tflops(name)
                kernels[name]["ceiling_tflops"] = round(c, 1)
                kernels[name]["frac_of_ceiling"] = round(rate / 1e12 / c, 4)
        else:
            kernels[name] = {"avg_us": round(avg_ms * 1e3, 2), "launches": n, "bound": "hbm",
                             "gbps": round(rate / 1e9, 1),
                             "frac": round(rate / 1e9 / PEAK_HBM_GBPS, 4)}
    dom_avg_s = dom_ms / dom_n * 1e-3
    achieved = work[dom][1] / dom_avg_s / 1e12
    gemm_total_ms = sum(v[0] for v in gemms.values()) / args.steps
    gemm_flops = sum(work[k][1] * (v[1] / args.steps) for k, v in gemms.items())

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "step_ms": step_stats(step_ms),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}_fwd_bwd", "T": wl.T, "D": wl.D, "I": wl.I, "E": wl.E,
                   "K": wl.K, "routing": "softmax_topk_renorm" if wl.score == 0 else "sigmoid",
                   "seed": wl.seed},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic(dom, wl.name),
                     # the kernel's attainable roof min(peak, AI x 8 TB/s) with its
                     # unavoidable HBM bytes, and the fraction of it achieved
                     "min_bytes": min_bytes[dom], "ceiling": round(ceiling_tflops(dom), 1),
                     "frac_of_ceiling": round(achieved / ceiling_tflops(dom), 4)},
        **extra,
        "router": router,
        "gemm_tflops_all": round(gemm_flops / (gemm_total_ms * 1e-3) / 1e12, 2),
        "gemm_frac_all": round(gemm_flops / (gemm_total_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
    }
    if args.cpu_tokens > 0:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, data, args.cpu_tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
