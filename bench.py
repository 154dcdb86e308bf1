#!/usr/bin/env python3
"""Benchmark one deterministic MoE layer step on one MI355X.

A step is the whole hot path on one batch: router top-k, schedule table,
forward (FC1+SwiGLU, FC2, combine) and backward (dH + SwiGLU-bwd + d-gate,
router backward, dX, dX reduce, dW2, dW1, dWr). Inputs are seeded synthetic
tensors of the workload's shapes, resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config kimi_k2_bf16]

With --config kimi_k2_mxfp8_stream a step is the streamed MXFP8 step: 8 micro-batches
of 2048 tokens (route, schedule, forward for 0..7, then backward for 7..0 through a
2-slot ring, weight gradients deferred to the last call). The expert weights are
quantised to their four MXFP8 orientations once, before timing (a per-weight-update
cost); activation and gradient quantisation is inside the step. --gemm mxfp4 runs the
same streamed step with MXFP4 (E2M1) expert GEMMs.

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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "mxfp8": 5000.0, "mxfp4": 10100.0}
MX_ELEM_BYTES = {"mxfp8": 1.0 + 1.0 / 32.0, "mxfp4": 0.5 + 1.0 / 32.0}  # element + its share of the scale byte
HBM_PEAK_GBS = 8000.0
GEMMS = ("fc1", "fc2", "dh", "dx", "dw2", "dw1")
FUSED = ("forward_fused", "backward_fused")  # whole passes in one persistent launch (their GEMMs and the rest)
# Compulsory-work bound of one whole step (ms): the larger of the expert-GEMM flops at the
# dense MFMA peak and the compulsory HBM bytes (weights once per pass, or once per
# micro-batch when streamed; activations once) at 8 TB/s. 2048-token bf16 steps: 0.46 GB
# -> 0.058 ms; Kimi-K2 bf16: 34.6 TFLOP (13.9 ms) against 121 GB (15.1 ms); streamed
# MXFP8: 328 GB of weight re-reads and activations -> 41 ms; the same step with MXFP4
# weights: the 245 GB of E4M3 weight re-reads become 245 * (0.5 + 1/32) / (1 + 1/32) =
# 126 GB, the other 83 GB stay -> 209 GB, 26.2 ms. The 64-token fp32 step is bound by
# launch latency and has none.
STEP_ROOFLINE_MS = {"small_bf16": 0.058, "imbalanced_bf16": 0.058, "kimi_k2_bf16": 15.1,
                    "kimi_k2_mxfp8_stream": 41.0, "kimi_k2_mxfp8_stream/mxfp4": 26.2}


def copy_ceiling_gbs(torch):
    """Measured HBM ceiling: a 1 GiB device-to-device copy (bytes read + written over its
    best time of three)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = None
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        best = t if best is None else min(best, t)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / (best * 1e-3) / 1e9


HBM_KERNELS = ("route", "schedule", "combine", "router_bwd", "dx_reduce", "gather", "dwr")


def hbm_kernels(w, per, copy_gbs):
    """The bandwidth-bound kernels of the step: algorithmic bytes per step over their
    summed time in the per-kernel breakdown, against 8 TB/s and against the measured
    copy ceiling. (Streamed MX steps: the per-micro-batch kernels only.)"""
    M = max(1, w.micro_batches)
    out = {"copy_ceiling_gbs": round(copy_gbs, 1)}
    for name in HBM_KERNELS:
        if name not in per or per[name] <= 0 or (M > 1 and name in ("dwr", "gather")):
            continue
        nb = kernel_work(w, name)[1] * M
        gbs = nb / (per[name] * 1e-3) / 1e9
        out[name] = {"ms": round(per[name], 4), "gb": round(nb / 1e9, 4), "gbs": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 3), "frac_of_copy": round(gbs / copy_gbs, 3)}
    return out


def launch_flops(w, name):
    """Flops of one launch of an expert GEMM (row GEMMs: one micro-batch; dW: the step)."""
    M = max(1, w.micro_batches)
    R = (w.T // M) * w.k
    per_row = {"fc1": 4, "fc2": 2, "dh": 2, "dx": 4, "dw2": 2 * M, "dw1": 4 * M,
               "forward_fused": 6, "backward_fused": 12}[name]
    return per_row * R * w.H * w.I


def launches_per_step(w, name):
    return 1 if name.startswith("dw") else max(1, w.micro_batches)


def kernel_work(w, name, active_experts=None):
    """Algorithmic work of one launch: ('mfma', flops) or ('hbm', bytes).

    Row GEMMs and the bandwidth kernels process one micro-batch per launch (the whole
    batch when there is one); the weight-gradient GEMMs process the whole step. For the
    MXFP8 row GEMMs the bound is the larger of flops / 5 PFLOP/s and bytes / 8 TB/s,
    bytes = the E4M3+E8M0 weights of the experts with rows (read once) plus the
    activation rows read and written."""
    M = max(1, w.micro_batches)
    T, H, I, E = w.T // M, w.H, w.I, w.E
    R = T * w.k
    es = 4 if w.act == "f32" else 2
    flops = {k: launch_flops(w, k) for k in GEMMS + FUSED}
    if w.gemm in MX_ELEM_BYTES and name in ("fc1", "fc2", "dh", "dx"):
        q = MX_ELEM_BYTES[w.gemm]
        ae = E if active_experts is None else active_experts
        wbytes = {"fc1": 2 * I * H, "fc2": H * I, "dh": I * H, "dx": H * 2 * I}[name] * q * ae
        act = {"fc1": T * H * q + R * (2 * I * 2 + I * 2 + I * q),
               "fc2": R * I * q + R * H * 2,
               "dh": T * H * q + R * (2 * I * 2 + I * 2 + 4) + R * (2 * I * 2 + 2 * I * q),
               "dx": R * 2 * I * q + R * H * 2}[name]
        b = wbytes + act
        if b / (HBM_PEAK_GBS * 1e9) > flops[name] / (MFMA_PEAK_TFLOPS[w.gemm] * 1e12):
            return "hbm", b
        return "mfma", flops[name]
    if name in flops:
        return "mfma", flops[name]
    nbytes = {"combine": R * H * es + T * H * es + 4 * R,
              # each slot's router-weight row is read from cache: Wr counts once
              "dx_reduce": R * H * es + T * H * es + 8 * R + E * H * es,
              # bf16: dWr also writes the routed-order x rows that dW1 reads
              "dwr": R * H * es + E * H * es + 8 * R + (R * H * es if w.act == "bf16" else 0),
              "gather": 2 * R * H * es + 8 * R,  # routed-order dO = g*dY rows for dW2
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
    if w.gemm in ("mxfp8", "mxfp4"):
        fmt = "e2m1" if w.gemm == "mxfp4" else "e4m3"
        fwd = oracle.mx.forward_mx(x, W, idx, g, w.E, w.I, fmt=fmt)
        oracle.mx.backward_mx(x, W, wr, idx, g, fwd, dy, w.I, fmt=fmt)
    else:
        fwd = oracle.forward(x, W, idx, g, w.act, w.E, w.I)
        oracle.backward(x, W, wr, idx, g, fwd, dy, w.act, w.I)
    dt = time.perf_counter() - t0
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cores = max(blas, len(os.sched_getaffinity(0)))
    return dt, cores, int(np.asarray(idx).size)


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="kimi_k2_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = per-workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile-m", type=int, default=0, help="schedule tile rows (0 = the library's two-wave rule)")
    ap.add_argument("--fused", action="store_true",
                    help="one persistent launch per pass (bf16, 32-row schedule tiles)")
    ap.add_argument("--replay", action="store_true",
                    help="forward-activation replay: keep no activations, form them again in the backward")
    ap.add_argument("--gemm", choices=["mxfp8", "mxfp4"], default=None,
                    help="element format of the MX expert GEMMs of an MX workload (default: the workload's)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (known bytes, for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer step; the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_stable_amd import inputs, mok

    w = inputs.WORKLOADS[args.config]
    if args.gemm is not None:
        if w.gemm not in ("mxfp8", "mxfp4"):
            print("--gemm applies to the MX workloads only", file=sys.stderr)
            sys.exit(2)
        w = inputs.replace(w, gemm=args.gemm)
    mx = w.gemm in ("mxfp8", "mxfp4")
    torch.cuda.set_device(0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    copy_gbs = copy_ceiling_gbs(torch)
    ntok = args.cpu_tokens or {"tiny_fp32": 64, "small_bf16": 2048, "imbalanced_bf16": 2048,
                               "kimi_k2_mxfp8_stream": 1}.get(w.name, 6)
    keep = cpu_sample_plan(w, ntok) if not args.no_cpu_baseline else []
    t0 = time.time()
    x, dy, wr, bias, w1, w2, kept = make_inputs(w, set(keep))
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.time() - t0))

    if mx:
        M = w.micro_batches
        d = mok.Desc(w.T // M, w.H, w.E, w.k, w.I, act=mok.BF16, gemm=mok.DTYPES[w.gemm], tile_m=args.tile_m, mb_count=M,
                     ring=2, flags=mok.FLAG_REPLAY if args.replay else 0)
        q = mok.MxWeights(d, "cuda")
        mok.weights_quantize(d, w1, w2, q)
        torch.cuda.synchronize()
        del w1, w2
        w1 = w2 = None
        torch.cuda.empty_cache()
        st = mok.StreamedStep(d, "cuda")

        def step():
            st.run(x, wr, bias, q, dy)
    else:
        d = mok.Desc(w.T, w.H, w.E, w.k, w.I, act=mok.DTYPES[w.act], tile_m=args.tile_m,
                     flags=(mok.FLAG_REPLAY if args.replay else 0) | (mok.FLAG_FUSED if args.fused else 0))
        buf = mok.Buffers(d, "cuda", backward=True)

        def step():
            mok.step(d, buf, x, wr, bias, w1, w2, dy=dy)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel breakdown from one traced (untimed) step
    with mok.KernelTrace("*", 512) as tr:
        step()
    per = {}
    for name, ms in tr.durations_ms():
        per[name] = per.get(name, 0.0) + ms
    dominant = max(per, key=per.get)
    log("per-kernel ms: " + ", ".join("%s %.3f" % kv for kv in sorted(per.items(), key=lambda kv: -kv[1])))

    # timed region; the dominant kernel's launches are bracketed by HIP events on its stream,
    # and every step by events of its own (median / min / max over the steps)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with mok.KernelTrace(dominant, capacity=max(16 * args.steps, 8)) as trd:
        start.record()
        evs[0].record()
        for i in range(args.steps):
            step()
            evs[i + 1].record()
        end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    each = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    step_stats = {"median": each[len(each) // 2] if len(each) % 2 else 0.5 * (each[len(each) // 2 - 1] + each[len(each) // 2]),
                  "min": each[0], "max": each[-1]}
    dom = [ms for _, ms in trd.durations_ms()]
    dom_ms = sum(dom) / len(dom)

    active = None
    if mx:  # experts with rows, averaged over the micro-batches (weights read by the row GEMMs)
        from mixture_experts_layer_stable_amd.mok import schedule_layout_query
        Ls = schedule_layout_query(d)
        active = sum(int((s[Ls["counts"]: Ls["counts"] + 4 * w.E].view(torch.int32) > 0).sum()) for s in st.sched)
        active /= len(st.sched)
    gdt = w.gemm if mx else w.act
    bound, work = kernel_work(w, dominant, active)
    if bound == "mfma":
        peak = MFMA_PEAK_TFLOPS[gdt]
        achieved = work / (dom_ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        peak = HBM_PEAK_GBS
        achieved = work / (dom_ms * 1e-3) / 1e9
        unit = "GB/s"
    traffic = measured_traffic(dominant, w.name) if args.gemm in (None, "mxfp8") else None
    rkey = w.name if args.gemm in (None, "mxfp8") else "%s/%s" % (w.name, args.gemm)
    gemm_ms = sum(per.get(k, 0.0) for k in GEMMS + FUSED)
    gemm_flops = sum(launches_per_step(w, k) * launch_flops(w, k) for k in GEMMS)
    mfma_util = 100.0 * gemm_flops / (gemm_ms * 1e-3) / (MFMA_PEAK_TFLOPS[gdt] * 1e12) if gemm_ms else None

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
        "dtype": gdt,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "k": w.k, "I": w.I,
                   "routing": "zipf-imbalanced" if w.zipf else "near-uniform", "tile_m": d.c().tile_m or "auto",
                   **({"activations": "replayed"} if args.replay else {}),
                   **({"launches": "one persistent kernel per pass"} if args.fused else {}),
                   **({"micro_batches": w.micro_batches, "ring_slots": 2, "gemm": w.gemm} if mx else {})},
        "roofline": {"bound": bound, "kernel": dominant, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic},
        "gemm_mfma_util_pct": mfma_util,
        "step_roofline": ({"ms": STEP_ROOFLINE_MS[rkey], "tokens_per_s": w.T / (STEP_ROOFLINE_MS[rkey] * 1e-3),
                           "frac": STEP_ROOFLINE_MS[rkey] / ms_step} if rkey in STEP_ROOFLINE_MS else None),
        "kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "step_ms": {k: round(v, 5) for k, v in step_stats.items()},
        "hbm_kernels": hbm_kernels(w, per, copy_gbs),
    }

    if not args.no_cpu_baseline:
        del x, dy, w1, w2
        torch.cuda.empty_cache()
        dt, cores, rows = cpu_baseline(w, ntok, kept)
        result["cpu_baseline"] = {
            "value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": "first %d of %d tokens (%d routed rows): oracle%s route + forward + backward, %.1f s" % (
                ntok, w.T, rows, " " + w.gemm.upper() if mx else "", dt)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
