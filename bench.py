#!/usr/bin/env python3
"""Benchmark one deterministic MoE layer step on one MI355X.

A step is the whole hot path on one batch: router top-k, schedule table,
forward (FC1+SwiGLU, FC2, combine) and backward (dH + SwiGLU-bwd + d-gate,
router backward, dX, dX reduce, dW2, dW1, dWr). Inputs are seeded synthetic
tensors of the workload's shapes, resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config kimi_k2_bf16]

Prints one JSON line. Runs on one GPU only; --gpus N > 1 exits with a message.
"""
import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/sec on 1 MI355X; grouped-GEMM MFMA util %"
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
GEMMS = ("fc1", "fc2", "dh", "dx", "dw2", "dw1")


def kernel_work(w, name):
    """Algorithmic work of one launch: ('mfma', flops) or ('hbm', bytes)."""
    R, H, I, T, E = w.R, w.H, w.I, w.T, w.E
    es = 4 if w.act == "f32" else 2
    flops = {"fc1": 4 * R * H * I, "fc2": 2 * R * H * I, "dh": 2 * R * H * I, "dx": 4 * R * H * I,
             "dw2": 2 * R * H * I, "dw1": 4 * R * H * I}
    if name in flops:
        return "mfma", flops[name]
    nbytes = {"combine": R * H * es + T * H * es + 4 * R,
              "dx_reduce": R * H * es + T * H * es + 8 * R + R * H * es,
              "dwr": R * H * es + E * H * es + 8 * R,
              "router_bwd": 4 * R * (I // 256 + 4),
              "route": T * H * es + E * H * es + 8 * R,
              "schedule": 4 * R * (2 * E // 64 + 2)}
    return "hbm", nbytes.get(name, 0)


def source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_layer_stable_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic_%s_%s.md" % (kernel, workload))
    if not os.path.exists(p):
        return None
    vals = {}
    for line in open(p):
        if line.startswith("<!-- ") and "=" in line:
            k, v = line[5:].split("-->")[0].strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash() or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def make_inputs(w, keep_experts=()):
    import torch
    from mixture_experts_layer_stable_amd import inputs
    dev = "cuda"
    dt = torch.float32 if w.act == "f32" else torch.bfloat16
    x = inputs.make_x(w).to(dev)
    dy = inputs.make_dy(w).to(dev)
    wr = inputs.make_wr(w).to(dev)
    b = inputs.make_bias(w)
    bias = None if b is None else b.to(dev)
    w1 = torch.empty(w.E, 2 * w.I, w.H, dtype=dt, device=dev)
    w2 = torch.empty(w.E, w.H, w.I, dtype=dt, device=dev)
    kept = {}
    for e in range(w.E):
        a1 = inputs.make_w1(w, e)
        a2 = inputs.make_w2(w, e)
        w1[e].copy_(a1)
        w2[e].copy_(a2)
        if e in keep_experts:
            kept[e] = (a1, a2)
    return x, dy, wr, bias, w1, w2, kept


def cpu_sample_plan(w, ntok):
    """Oracle routing of the first ntok tokens (to know which experts' weights to keep)."""
    import oracle
    from mixture_experts_layer_stable_amd import inputs
    x = inputs.make_x(w, 0, ntok).float().numpy()
    wr = inputs.make_wr(w).float().numpy()
    b = inputs.make_bias(w)
    _, idx, _ = oracle.route(x, wr, w.k, None if b is None else b.numpy())
    return sorted(set(idx.ravel().tolist()))


class KeptWeights:
    def __init__(self, kept):
        self.kept = kept

    def w1(self, e):
        return self.kept[e][0].float().numpy().astype("float64")

    def w2(self, e):
        return self.kept[e][1].float().numpy().astype("float64")


def cpu_baseline(w, ntok, kept):
    """The oracle, as it stands, on the first ntok tokens: route, forward, backward."""
    import numpy as np
    import oracle
    from mixture_experts_layer_stable_amd import inputs
    from threadpoolctl import threadpool_info
    x = inputs.make_x(w, 0, ntok).float().numpy()
    dy = inputs.make_dy(w, 0, ntok).float().numpy()
    wr = inputs.make_wr(w).float().numpy()
    b = inputs.make_bias(w)
    b = None if b is None else b.numpy()
    W = KeptWeights(kept)
    t0 = time.perf_counter()
    _, idx, g = oracle.route(x, wr, w.k, b)
    fwd = oracle.forward(x, W, idx, g, w.act, w.E, w.I)
    oracle.backward(x, W, wr, idx, g, fwd, dy, w.act, w.I)
    dt = time.perf_counter() - t0
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cores = max(blas, len(os.sched_getaffinity(0)))
    return dt, cores, int(np.asarray(idx).size)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="kimi_k2_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = per-workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (known bytes, for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer step; multi-GPU runs (--gpus %d) are not part of "
              "this build" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_stable_amd import inputs, mok

    w = inputs.WORKLOADS[args.config]
    if w.gemm == "mxfp8":
        print("workload %s (MXFP8 expert GEMMs) is not implemented by this version" % w.name, file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ntok = args.cpu_tokens or {"tiny_fp32": 64, "small_bf16": 512, "imbalanced_bf16": 512}.get(w.name, 6)
    keep = cpu_sample_plan(w, ntok) if not args.no_cpu_baseline else []
    t0 = time.time()
    x, dy, wr, bias, w1, w2, kept = make_inputs(w, set(keep))
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.time() - t0))

    d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.DTYPES[w.act])
    buf = mok.Buffers(d, "cuda", backward=True)

    def step():
        mok.step(d, buf, x, wr, bias, w1, w2, dy=dy)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel breakdown from one traced (untimed) step
    with mok.KernelTrace("*", 64) as tr:
        step()
    per = {}
    for name, ms in tr.durations_ms():
        per[name] = per.get(name, 0.0) + ms
    dominant = max(per, key=per.get)
    log("per-kernel ms: " + ", ".join("%s %.3f" % kv for kv in sorted(per.items(), key=lambda kv: -kv[1])))

    # timed region; the dominant kernel's launches are bracketed by HIP events on its stream
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with mok.KernelTrace(dominant, capacity=max(4 * args.steps, 8)) as trd:
        start.record()
        for _ in range(args.steps):
            step()
        end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    dom = [ms for _, ms in trd.durations_ms()]
    dom_ms = sum(dom) / len(dom)

    bound, work = kernel_work(w, dominant)
    if bound == "mfma":
        peak = MFMA_PEAK_TFLOPS[w.act]
        achieved = work / (dom_ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        peak = HBM_PEAK_GBS
        achieved = work / (dom_ms * 1e-3) / 1e9
        unit = "GB/s"
    traffic = measured_traffic(dominant, w.name)
    gemm_ms = sum(per.get(k, 0.0) for k in GEMMS)
    gemm_flops = sum(kernel_work(w, k)[1] for k in GEMMS)
    mfma_util = 100.0 * gemm_flops / (gemm_ms * 1e-3) / (MFMA_PEAK_TFLOPS[w.act] * 1e12) if gemm_ms else None

    result = {
        "metric": METRIC,
        "value": w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "k": w.k, "I": w.I,
                   "routing": "zipf-imbalanced" if w.zipf else "near-uniform"},
        "roofline": {"bound": bound, "kernel": dominant, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic},
        "gemm_mfma_util_pct": mfma_util,
        "kernel_ms": {k: round(v, 4) for k, v in per.items()},
    }

    if not args.no_cpu_baseline:
        del x, dy, w1, w2, buf
        torch.cuda.empty_cache()
        dt, cores, rows = cpu_baseline(w, ntok, kept)
        result["cpu_baseline"] = {
            "value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d tokens (%d routed rows): oracle route + forward + backward, %.1f s" % (
                ntok, w.T, rows, dt)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
